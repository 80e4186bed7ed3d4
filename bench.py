"""Throughput of the row-typed Q_q projection (libqalg) on one MI355X.

Workload (one step): the dense-model FFN shape (D, F) = (4096, 12288) in bf16
with q = 8 (512 x 1536 weight blocks), M = 16384 token rows at positions
0..M-1, types tau(p) = p mod 8:
    type schedule (positions -> tau), type index, then the up projection
    X_up [M, 4096] x W_up [4096, 12288] and the down projection
    X_dn [M, 12288] x W_dn [12288, 4096], both forward, fp32 accumulation.
Inputs are seeded synthetic N(0,1) activations and N(0,1/K) weights, resident
in HBM before timing starts.  Before the W warm-up steps the step runs untimed
for --prewarm-s seconds (the clock ramp from idle takes about 25 ms of load);
then exactly K steps are timed with HIP events on the launch stream.

Reported (one JSON line):
  value            algebra TFLOP/s of the step: 2 * rho_q * M*K*N per projection
                   (rho_q = (2q-1)/q^2, eq 21 and eq 24 of arXiv 2609.32814)
  frac_peak        value / 2516.6 TFLOP/s (MI355X dense bf16 MFMA)
  dense_equiv_tflops  2*M*K*N per projection / step time
  speedup_vs_dense t(same kernel template at q = 1, i.e. a plain dense GEMM) / t(q)
  roofline         the forward GEMM kernel against the bf16 MFMA peak, its
                   launch time taken with HIP events on the launch stream
  cpu_baseline     the fp64 CPU oracle on the host cores (a bounded sample)
  protocol         the pages' timing protocol on the two forwards: graph replays of at
                   least 2 ms per trial, 12 trials alternating q = 8 and its q = 1 control,
                   medians and interquartile ranges, and a flushed (cold-cache) run
  clock            the shader clock sampled during back-to-back replays of the up forward,
                   and the bf16 MFMA peak at that clock (256 CU x f x 4096 FLOP)
  extra            further legs, each timed separately: the ~110M-LM FFN (768 <-> 3072,
                   q = 4, M = 8192, both roofline fractions), training (forward + dX +
                   dW at the same shape), small-M decode (64 experts), gated
                   SwiGLU FFN (forward and training step), the 64-expert shapes at
                   M = 1..1024 against q = 1, the pilot FFN under
                   Q_2^(x)2 / Q_4 / q = 1, few rows per type (q = 32), algebraic
                   attention (prefill, and cached decoding against a 4096-slot cache),
                   the graph law Q_G and unequal group widths (forward,
                   dX, dW each)
"""
from __future__ import annotations

import argparse
import json
import os
import pathlib
import sys
import time
from concurrent.futures import ThreadPoolExecutor

ROOT = pathlib.Path(__file__).resolve().parent
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))

PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 bf16 FLOP/clk/CU (dense)
PEAK_HBM_GBS = 8000.0

WORKLOAD = "ffn_up_down_D4096_F12288_q8_M16384_bf16_fwd"
M, D, F, QQ = 16384, 4096, 12288, 8


def rho(q: int) -> float:
    return (2 * q - 1) / (q * q)


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


class Protocol:
    """The pages' timing protocol (App E, App F), adapted: each operation is captured in a HIP
    graph and replayed until a timed trial lasts at least 2 ms (warm caches); trials alternate
    between the algebra and its q = 1 control of the same template, 12 of each, reported as
    median and interquartile range; a flushed run writes then reads a 1 GiB buffer before each
    single replay (outside the timed interval), so that neither L2 nor the 256 MB MALL holds
    the operands and no dirty lines of the flush are written back inside it."""

    def __init__(self, torch, np, dev):
        self.torch, self.np = torch, np
        self.flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        self.side = torch.cuda.Stream()   # default priority

    def capture(self, fn):
        """fn(stream) enqueues the operation; it is run once eagerly (first-call set-up), then captured."""
        torch = self.torch
        self.side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(self.side):
            fn(self.side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=self.side):
            fn(self.side)
        torch.cuda.synchronize()
        return g

    def _events(self):
        E = self.torch.cuda.Event
        return E(enable_timing=True), E(enable_timing=True)

    def replay_ms(self, g, reps):
        a, b = self._events()
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        self.torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    def flushed_ms(self, g, n=8):
        np, out = self.np, []
        for k in range(n + 2):
            self.flush.fill_(k & 0xFF)
            self.flush.view(self.torch.float32).sum()
            out.append(self.replay_ms(g, 1))
        return float(np.median(out[2:]))

    def stats(self, xs):
        np = self.np
        q25, q50, q75 = np.percentile(xs, [25, 50, 75])
        return {"median_ms": round(float(q50), 5), "iqr_ms": [round(float(q25), 5), round(float(q75), 5)]}

    def compare(self, g_q, g_1, trials=12, min_ms=2.0, flushed=True):
        """Alternating warm trials of the algebra (g_q) and its q = 1 control (g_1), then flushed runs."""
        np = self.np
        for g in (g_q, g_1):      # settle the clock on this operation
            self.replay_ms(g, 20)
        reps = {id(g): max(1, int(np.ceil(min_ms / self.replay_ms(g, 3)))) for g in (g_q, g_1)}
        tq, t1 = [], []
        for _ in range(trials):
            tq.append(self.replay_ms(g_q, reps[id(g_q)]))
            t1.append(self.replay_ms(g_1, reps[id(g_1)]))
        res = {"warm": self.stats(tq), "warm_q1": self.stats(t1), "replays_per_trial": [reps[id(g_q)], reps[id(g_1)]],
               "trials": trials}
        res["speedup_vs_q1"] = round(float(np.median(t1) / np.median(tq)), 3)
        if flushed:
            fq, f1 = self.flushed_ms(g_q), self.flushed_ms(g_1)
            res["flushed_ms"], res["flushed_q1_ms"] = round(fq, 5), round(f1, 5)
            res["flushed_speedup_vs_q1"] = round(f1 / fq, 3)
        return res


def sclk_sampler(torch):
    """A function returning the shader clock (MHz) of GPU 0, or None when no source is visible:
    the hwmon node of the GPU's PCI device, else its pp_dpm_sclk table (the entry marked '*' is
    the current clock).  The card is found by its PCI address."""
    import glob
    import re
    try:
        pr = torch.cuda.get_device_properties(0)
        dom, bus, devn = (getattr(pr, "pci_domain_id", 0), getattr(pr, "pci_bus_id", None),
                          getattr(pr, "pci_device_id", 0))
        if bus is None:
            return None
        node = f"/sys/bus/pci/devices/{dom:04x}:{bus:02x}:{devn:02x}.0"
        hw = glob.glob(f"{node}/hwmon/hwmon*/freq1_input")
        dpm = glob.glob(f"{node}/pp_dpm_sclk")

        def read_hwmon():
            try:
                with open(hw[0]) as f:
                    return int(f.read().strip()) / 1e6
            except (OSError, ValueError):
                return None

        def read_dpm():
            try:
                with open(dpm[0]) as f:
                    for line in f:
                        if line.rstrip().endswith("*"):
                            m = re.search(r"(\d+)\s*Mhz", line, re.I)
                            return float(m.group(1)) if m else None
            except OSError:
                return None
            return None
        for read in ((read_hwmon,) if hw else ()) + ((read_dpm,) if dpm else ()):
            if read() is not None:
                read.source = "hwmon freq1_input" if read is read_hwmon else "pp_dpm_sclk (current entry)"
                return read
        return None
    except Exception:  # informational only
        return None


def sustained_clock(torch, np, g, seconds=0.4):
    """Median shader clock sampled every ~5 ms while graph g is replayed back to back for `seconds`."""
    import threading
    read = sclk_sampler(torch)
    if read is None:
        return None
    vals, stop = [], threading.Event()

    def sample():
        while not stop.is_set():
            v = read()
            if v:
                vals.append(v)
            time.sleep(0.005)
    th = threading.Thread(target=sample)
    t_end = time.time() + seconds
    th.start()
    while time.time() < t_end:
        for _ in range(10):
            g.replay()
        torch.cuda.synchronize()
    stop.set()
    th.join()
    if not vals:
        return None
    f = float(np.median(vals))
    return {"sclk_mhz_median": round(f, 1), "samples": len(vals),
            "peak_at_clock_tflops": round(256 * f * 1e6 * 4096 / 1e12, 1),
            "source": f"{read.source} of the GPU's PCI device, sampled during back-to-back replays"}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--prewarm-s", type=float, default=0.3,
                    help="untimed steps run for this wall time before the warm-up steps (clock ramp from idle)")
    ap.add_argument("--cpu-rows", type=int, default=16384,
                    help="rows of each projection the CPU oracle leg evaluates")
    ap.add_argument("--cpu-rows-1t", type=int, default=1024,
                    help="rows of each projection the one-thread CPU oracle run evaluates")
    ap.add_argument("--no-extra", action="store_true", help="skip the training and decode legs")
    ap.add_argument("--no-dense", action="store_true", help="skip the protocol's q = 1 control trials")
    ap.add_argument("--legs", default="all", help="comma-separated extra legs to run (default: all)")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (scales HBM counters)")
    return ap.parse_args()


def main() -> int:
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the row-typed projection is benchmarked on a single MI355X", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import gemm_qalg_forward_amd as Q
    import synth

    Q.lib()  # fails loudly without the HIP library
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    # ---------------- inputs (seeded, synthetic; generated in parallel per operand) ----------------
    t0 = time.time()
    c = 3
    specs = {
        "Xu": (1000 * c + 1, (M, D), 1.0),
        "Wu": (1000 * c + 2, (D, F), D ** -0.5),
        "Xd": (1000 * c + 11, (M, F), 1.0),
        "Wd": (1000 * c + 12, (F, D), F ** -0.5),
    }
    with ThreadPoolExecutor(max_workers=4) as ex:
        futs = {k: ex.submit(synth.normal_operand, s, shp, std, "bf16") for k, (s, shp, std) in specs.items()}
        host = {k: f.result() for k, f in futs.items()}

    def to_dev(op):
        return torch.from_numpy(op.bits.view(np.int16)).view(torch.bfloat16).to(dev)

    d = {k: to_dev(v) for k, v in host.items()}
    pos = torch.from_numpy(synth.cyclic_positions(M)).to(dev)
    tau = torch.empty(M, dtype=torch.int32, device=dev)
    ws = Q.workspace(QQ, M, device=dev)
    Yu = torch.empty(M, F, dtype=torch.bfloat16, device=dev)
    Yd = torch.empty(M, D, dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] inputs ready in {time.time() - t0:.1f} s")

    ready = Q.QALG_FLAG_INDEX_READY

    def step(q, tau_t, ws_t, ev=None):
        Q.qalg_type_schedule(pos, q, Q.QALG_SCHEDULE_CYCLIC, 0, tau=tau_t, stream=stream)
        Q.qalg_build_index(tau_t, q, ws=ws_t, stream=stream)
        if ev is not None:
            ev[0].record(stream)
        Q.qalg_forward(d["Xu"], d["Wu"], tau_t, q, Y=Yu, ws=ws_t, flags=ready, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        Q.qalg_forward(d["Xd"], d["Wd"], tau_t, q, Y=Yd, ws=ws_t, flags=ready, stream=stream)
        if ev is not None:
            ev[2].record(stream)

    def prewarm(q, tau_t, ws_t, seconds):
        # From idle the GPU needs about 25 ms of sustained load before its clock
        # settles (per-launch times fall from 0.8 to 0.36 ms over the first
        # ~50 launches, then stay flat), which a handful of warm-up steps does
        # not cover: run the untimed step for a fixed wall time first.
        t_end = time.time() + seconds
        while time.time() < t_end:
            for _ in range(10):
                step(q, tau_t, ws_t)
            torch.cuda.synchronize()

    def timed(q, tau_t, ws_t, steps, warmup, prewarm_s=0.0):
        if prewarm_s > 0:
            prewarm(q, tau_t, ws_t, prewarm_s)
        for _ in range(warmup):
            step(q, tau_t, ws_t)
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for k in range(steps):
            step(q, tau_t, ws_t, evs[k])
        end.record(stream)
        torch.cuda.synchronize()
        total_ms = start.elapsed_time(end)
        up = [e[0].elapsed_time(e[1]) for e in evs]
        dn = [e[1].elapsed_time(e[2]) for e in evs]
        return total_ms, up, dn

    # ---------------- the step at q = 8 ----------------
    total_ms, up_ms, dn_ms = timed(QQ, tau, ws, args.steps, args.warmup, args.prewarm_s)
    ms_step = total_ms / args.steps
    alg_flop_proj = 2.0 * rho(QQ) * M * D * F
    dense_flop_proj = 2.0 * M * D * F
    step_alg = 2 * alg_flop_proj
    value = step_alg / (ms_step * 1e-3) / 1e12
    fwd_launch_ms = (sum(up_ms) + sum(dn_ms)) / (len(up_ms) + len(dn_ms))
    achieved = alg_flop_proj / (fwd_launch_ms * 1e-3) / 1e12
    log(f"[bench] q=8 step {ms_step:.3f} ms; forward launch up {np.median(up_ms):.3f} ms "
        f"down {np.median(dn_ms):.3f} ms; {value:.1f} algebra TFLOP/s")

    # ---------------- the pages' protocol: graph replays, alternating q = 8 / q = 1 trials ----------------
    # (the dense control is the same kernel template at q = 1, where Q_1 is the plain product)
    proto = Protocol(torch, np, dev)
    tau1 = torch.zeros(M, dtype=torch.int32, device=dev)
    ws1 = Q.workspace(1, M, device=dev)
    Q.qalg_build_index(tau1, 1, ws=ws1, stream=stream)
    torch.cuda.synchronize()
    graphs = {
        (proj, q): proto.capture(lambda st, X=X, W=W, Y=Y, q=q, t=t, w=w: Q.qalg_forward(
            X, W, t, q, Y=Y, ws=w, flags=ready, stream=st))
        for proj, X, W, Y in (("up", d["Xu"], d["Wu"], Yu), ("down", d["Xd"], d["Wd"], Yd))
        for q, t, w in ((QQ, tau, ws), (1, tau1, ws1))
    }
    protocol = {}
    speedup = dense_tflops = None
    if not args.no_dense:
        protocol = {proj: proto.compare(graphs[(proj, QQ)], graphs[(proj, 1)]) for proj in ("up", "down")}
        t8 = sum(protocol[p_]["warm"]["median_ms"] for p_ in ("up", "down"))
        t1 = sum(protocol[p_]["warm_q1"]["median_ms"] for p_ in ("up", "down"))
        speedup = round(t1 / t8, 3)
        dense_tflops = round(2 * dense_flop_proj / (t1 * 1e-3) / 1e12, 1)
        for p_ in ("up", "down"):
            r_ = protocol[p_]
            r_["algebra_tflops_warm"] = round(alg_flop_proj / (r_["warm"]["median_ms"] * 1e-3) / 1e12, 1)
            r_["algebra_tflops_flushed"] = round(alg_flop_proj / (r_["flushed_ms"] * 1e-3) / 1e12, 1)
            r_["dense_tflops_q1_warm"] = round(dense_flop_proj / (r_["warm_q1"]["median_ms"] * 1e-3) / 1e12, 1)
        log(f"[bench] protocol (12 alternating trials, graph replays >= 2 ms): {protocol}")
        log(f"[bench] q=1 dense template: {dense_tflops:.1f} TFLOP/s; speedup {speedup:.2f}x")
    clock = sustained_clock(torch, np, graphs[("up", QQ)])
    if clock is not None:
        clock["frac_of_peak_at_clock"] = round(achieved / clock["peak_at_clock_tflops"], 4)
    log(f"[bench] sustained clock during the up forward: {clock}")

    extra = {}
    legs = {
        "lm_ffn_q4": lambda: lm_ffn_leg(Q, torch, np, synth, dev, proto),
        "training": lambda: training_leg(Q, torch, np, synth, dev, stream),
        "decode": lambda: decode_leg(Q, torch, np, synth, dev, stream),
        "experts": lambda: experts_leg(Q, torch, np, synth, dev, stream),
        "gated_ffn": lambda: gated_leg(Q, torch, np, synth, dev, stream),
        "pilot_ffn": lambda: pilot_leg(Q, torch, np, synth, dev, stream),
        "few_rows": lambda: few_rows_leg(Q, torch, np, synth, dev, stream),
        "attention": lambda: attention_leg(Q, torch, np, synth, dev, stream),
        "attention_decode": lambda: attention_decode_leg(Q, torch, np, synth, dev, proto),
        "graph_law": lambda: graph_leg(Q, torch, np, synth, dev, stream),
        "unequal_widths": lambda: widths_leg(Q, torch, np, synth, dev, stream),
    }
    chosen = [] if args.no_extra else (list(legs) if args.legs == "all" else args.legs.split(","))
    for name in chosen:
        if name not in legs:
            raise SystemExit(f"unknown leg {name!r}; choose from {', '.join(legs)}")
        extra[name] = legs[name]()

    if args.copy_calib_mib > 0:
        n = args.copy_calib_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: {n} bytes read, {n} bytes written")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_leg(np, host, args.cpu_rows)
        cpu["one_thread"] = cpu_leg(np, host, args.cpu_rows_1t, threads=1)

    out = {
        "metric": "algebra TFLOP/s + % bf16 MFMA peak; speedup vs same-shape dense GEMM",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "M": M, "D": D, "F": F, "q": QQ,
                   "tau": "p mod 8, p = 0..M-1", "ops": ["type_schedule", "type_index",
                                                        "forward up", "forward down"]},
        "frac_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "dense_equiv_tflops": round(2 * dense_flop_proj / (ms_step * 1e-3) / 1e12, 1),
        "speedup_vs_dense": speedup,
        "dense_template_tflops": dense_tflops,
        "protocol": protocol,
        "clock": clock,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": profiled_traffic(),
                     "kernel": "fwd_persistent_kernel (forward GEMM, 256x256 tiles)",
                     "per_launch_flop": alg_flop_proj, "launch_ms": round(fwd_launch_ms, 4)},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(out), flush=True)
    return 0


PROFILE = ROOT / "profiles" / "fwd_persistent_ffn_D4096_F12288_q8_M16384.md"


def profiled_traffic():
    """HBM bytes per forward launch from the committed rocprofv3 counter summary
    (FETCH_SIZE x2 + WRITE_SIZE x1, scaled against a plain 1 GiB copy), or None
    when the kernel source changed since the counters were taken."""
    import hashlib
    try:
        fields = {}
        for line in PROFILE.read_text().splitlines():
            if ":" in line and not line.startswith(("#", "|", " ")):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
        src = ROOT / fields["kernel_source"]
        if hashlib.sha256(src.read_bytes()).hexdigest() != fields["kernel_source_sha256"]:
            return None
        return int(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def lm_ffn_leg(Q, torch, np, synth, dev, proto):
    """The ~110M-LM FFN shapes in bf16 with q = 4: up 768 -> 3072 and down 3072 -> 768, M = 8192
    (8 sequences x 1024 positions, tau = (m mod 1024) mod 4), forward.  At these sizes a launch
    lasts about 10 us, so each projection is timed with the graph-replay protocol (warm, and
    flushed), against the q = 1 control.  The arithmetic intensity (about 250 FLOP per algorithmic
    byte) sits just under the ridge of the MFMA and HBM roofs, so both fractions are reported."""
    c, Mx, q = 2, 8192, 4
    to = lambda op: torch.from_numpy(op.bits.view(np.int16)).view(torch.bfloat16).to(dev)  # noqa: E731
    pos = synth.cyclic_positions(Mx, seq_len=1024)
    tau = Q.qalg_type_schedule(torch.from_numpy(pos).to(dev), q)
    tau1 = torch.zeros(Mx, dtype=torch.int32, device=dev)
    ws, ws1 = Q.workspace(q, Mx, device=dev), Q.workspace(1, Mx, device=dev)
    Q.qalg_build_index(tau, q, ws=ws)
    Q.qalg_build_index(tau1, 1, ws=ws1)
    r = Q.QALG_FLAG_INDEX_READY
    res = {"workload": "lm_ffn_q4_M8192_bf16_fwd", "tau": "(m mod 1024) mod 4"}
    for proj, K, N, off in (("up", 768, 3072, 0), ("down", 3072, 768, 10)):
        X = to(synth.normal_operand(1000 * c + 1 + off, (Mx, K), 1.0, "bf16"))
        W = to(synth.normal_operand(1000 * c + 2 + off, (K, N), K ** -0.5, "bf16"))
        Y = torch.empty(Mx, N, dtype=torch.bfloat16, device=dev)
        g_q = proto.capture(lambda st: Q.qalg_forward(X, W, tau, q, Y=Y, ws=ws, flags=r, stream=st))
        g_1 = proto.capture(lambda st: Q.qalg_forward(X, W, tau1, 1, Y=Y, ws=ws1, flags=r, stream=st))
        cmp_ = proto.compare(g_q, g_1)
        flop = 2.0 * rho(q) * Mx * K * N
        byts = 2 * (Mx * K + K * N + Mx * N)
        for key, t in (("warm", cmp_["warm"]["median_ms"]), ("flushed", cmp_["flushed_ms"])):
            tf = flop / (t * 1e-3) / 1e12
            gbs = byts / (t * 1e-3) / 1e9
            cmp_[f"{key}_algebra_tflops"] = round(tf, 1)
            cmp_[f"{key}_frac_mfma"] = round(tf / PEAK_BF16_TFLOPS, 4)
            cmp_[f"{key}_GBs"] = round(gbs, 1)
            cmp_[f"{key}_frac_hbm"] = round(gbs / PEAK_HBM_GBS, 4)
        cmp_["algebra_flop"] = flop
        cmp_["algorithmic_bytes"] = byts
        res[proj] = cmp_
        del X, W, Y, g_q, g_1
    log(f"[bench] 110M-LM FFN leg: {res}")
    return res


def training_leg(Q, torch, np, synth, dev, stream):
    """Forward + dX + dW at (4096, 12288), q = 8, M = 16384 (the up projection's shape)."""
    c = 5
    X = synth.normal_operand(1000 * c + 1, (M, D), 1.0, "bf16")
    W = synth.normal_operand(1000 * c + 2, (D, F), D ** -0.5, "bf16")
    dY = synth.normal_operand(1000 * c + 3, (M, F), 1.0, "bf16")
    to = lambda op: torch.from_numpy(op.bits.view(np.int16)).view(torch.bfloat16).to(dev)  # noqa: E731
    Xd, Wd, dYd = to(X), to(W), to(dY)
    tau = torch.from_numpy((np.arange(M) % QQ).astype(np.int32)).to(dev)
    # with the dW scratch, dW splits the contraction of its diagonal tiles
    ws = Q.workspace(QQ, M, device=dev, dw_shape=(D, F))
    Y = torch.empty(M, F, dtype=torch.bfloat16, device=dev)
    dX = torch.empty(M, D, dtype=torch.bfloat16, device=dev)
    dW = torch.empty(D, F, dtype=torch.bfloat16, device=dev)
    Q.qalg_build_index(tau, QQ, ws=ws, stream=stream)
    r = Q.QALG_FLAG_INDEX_READY
    ops = {
        "fwd": lambda: Q.qalg_forward(Xd, Wd, tau, QQ, Y=Y, ws=ws, flags=r, stream=stream),
        "dx": lambda: Q.qalg_backward_dx(dYd, Wd, tau, QQ, dX=dX, ws=ws, flags=r, stream=stream),
        "dw": lambda: Q.qalg_backward_dw(Xd, dYd, tau, QQ, dW=dW, ws=ws, flags=r, stream=stream),
    }
    flop = 2.0 * rho(QQ) * M * D * F
    res = {"workload": "train_D4096_F12288_q8_M16384_bf16", "per_op_flop": flop}
    tot = 0.0
    for name, fn in ops.items():
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n = 5
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / n
        tot += ms
        res[f"{name}_ms"] = round(ms, 4)
        res[f"{name}_tflops"] = round(flop / (ms * 1e-3) / 1e12, 1)
    res["step_ms"] = round(tot, 4)
    res["step_tflops"] = round(3 * flop / (tot * 1e-3) / 1e12, 1)
    log(f"[bench] training leg: {res}")
    return res


def graph_leg(Q, torch, np, synth, dev, stream):
    """Graph law Q_G (section 3.1) at (4096, 12288), q = 8, M = 16384: forward, dX and dW on a seeded
    random digraph (each of the 56 edges kept with probability 1/2)."""
    c = 9
    X = synth.normal_operand(1000 * c + 1, (M, D), 1.0, "bf16")
    W = synth.normal_operand(1000 * c + 2, (D, F), D ** -0.5, "bf16")
    dY = synth.normal_operand(1000 * c + 3, (M, F), 1.0, "bf16")
    g = np.random.Generator(np.random.PCG64(1000 * c + 4))
    edges = [(a, b) for a in range(QQ) for b in range(QQ) if a != b and g.random() < 0.5]
    masks = [0] * QQ
    for a, b in edges:
        masks[a] |= 1 << b
    adj = torch.tensor(masks, dtype=torch.int64, device=dev)
    to = lambda op: torch.from_numpy(op.bits.view(np.int16)).view(torch.bfloat16).to(dev)  # noqa: E731
    Xd, Wd, dYd = to(X), to(W), to(dY)
    tau = torch.from_numpy((np.arange(M) % QQ).astype(np.int32)).to(dev)
    ws = Q.workspace(QQ, M, device=dev, dw_shape=(D, F))
    Y = torch.empty(M, F, dtype=torch.bfloat16, device=dev)
    dX = torch.empty(M, D, dtype=torch.bfloat16, device=dev)
    dW = torch.empty(D, F, dtype=torch.bfloat16, device=dev)
    Q.qalg_build_index(tau, QQ, ws=ws, stream=stream)
    r = Q.QALG_FLAG_INDEX_READY
    ops = {
        "fwd": lambda: Q.qalg_forward_graph(Xd, Wd, tau, QQ, adj, Y=Y, ws=ws, flags=r, stream=stream),
        "dx": lambda: Q.qalg_backward_dx_graph(dYd, Wd, tau, QQ, adj, dX=dX, ws=ws, flags=r, stream=stream),
        "dw": lambda: Q.qalg_backward_dw_graph(Xd, dYd, tau, QQ, adj, dW=dW, ws=ws, flags=r, stream=stream),
    }
    # a type-i row multiplies 1 + 2 outdeg(i) blocks of s x r (eq 10-11)
    blocks = sum(1 + 2 * bin(masks[i]).count("1") for i in range(QQ))
    flop = 2.0 * (M // QQ) * (D // QQ) * (F // QQ) * blocks
    res = {"workload": "graph_law_D4096_F12288_q8_M16384_random_half", "edges": len(edges),
           "per_op_flop": flop, "fraction_of_dense": round(blocks / QQ ** 3, 4)}
    for name, fn in ops.items():
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n = 5
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / n
        res[f"{name}_ms"] = round(ms, 4)
        res[f"{name}_tflops"] = round(flop / (ms * 1e-3) / 1e12, 1)
    log(f"[bench] graph-law leg: {res}")
    return res


def widths_leg(Q, torch, np, synth, dev, stream):
    """Unequal group widths (eq 18) at D = 4096 -> F = 12288, q = 4, M = 16384 (cyclic types): input
    widths 512 / 768 / 1024 / 1792, output widths three times those; forward, dX and dW."""
    c = 10
    kw = [512, 768, 1024, 1792]
    nw = [3 * w for w in kw]
    q = len(kw)
    X = synth.normal_operand(1000 * c + 1, (M, D), 1.0, "bf16")
    W = synth.normal_operand(1000 * c + 2, (D, F), D ** -0.5, "bf16")
    dY = synth.normal_operand(1000 * c + 3, (M, F), 1.0, "bf16")
    to = lambda op: torch.from_numpy(op.bits.view(np.int16)).view(torch.bfloat16).to(dev)  # noqa: E731
    Xd, Wd, dYd = to(X), to(W), to(dY)
    tau = torch.from_numpy((np.arange(M) % q).astype(np.int32)).to(dev)
    ws = Q.workspace(q, M, device=dev, dw_shape=(D, F))
    Y = torch.empty(M, F, dtype=torch.bfloat16, device=dev)
    dX = torch.empty(M, D, dtype=torch.bfloat16, device=dev)
    dW = torch.empty(D, F, dtype=torch.bfloat16, device=dev)
    Q.qalg_build_index(tau, q, ws=ws, stream=stream)
    r = Q.QALG_FLAG_INDEX_READY
    ops = {
        "fwd": lambda: Q.qalg_forward_widths(Xd, Wd, tau, q, kw, nw, Y=Y, ws=ws, flags=r, stream=stream),
        "dx": lambda: Q.qalg_backward_dx_widths(dYd, Wd, tau, q, kw, nw, dX=dX, ws=ws, flags=r, stream=stream),
        "dw": lambda: Q.qalg_backward_dw_widths(Xd, dYd, tau, q, kw, nw, dW=dW, ws=ws, flags=r, stream=stream),
    }
    # a type-i row: s_i N (its strip) + sum over j != i of s_j r_j (the diagonal blocks), eq 18
    macs_per_type = [kw[i] * F + sum(kw[j] * nw[j] for j in range(q) if j != i) for i in range(q)]
    flop = 2.0 * (M // q) * sum(macs_per_type)
    res = {"workload": "widths_D4096_F12288_q4_M16384_w512_768_1024_1792", "per_op_flop": flop,
           "fraction_of_dense": round(flop / (2.0 * M * D * F), 4)}
    for name, fn in ops.items():
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n = 5
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / n
        res[f"{name}_ms"] = round(ms, 4)
        res[f"{name}_tflops"] = round(flop / (ms * 1e-3) / 1e12, 1)
    log(f"[bench] unequal-widths leg: {res}")
    return res


def gated_leg(Q, torch, np, synth, dev, stream):
    """Gated (SwiGLU) FFN at (4096, 12288), q = 8, M = 16384: fused gate/up (silu(x W_g) * x W_u) + down."""
    c = 6
    X = synth.normal_operand(1000 * c + 1, (M, D), 1.0, "bf16")
    Wg = synth.normal_operand(1000 * c + 2, (D, F), D ** -0.5, "bf16")
    Wu = synth.normal_operand(1000 * c + 3, (D, F), D ** -0.5, "bf16")
    Wd = synth.normal_operand(1000 * c + 4, (F, D), F ** -0.5, "bf16")
    to = lambda op: torch.from_numpy(op.bits.view(np.int16)).view(torch.bfloat16).to(dev)  # noqa: E731
    Xd, Wdd = to(X), to(Wd)
    Wgu = Q.qalg_merge_gate_up(to(Wg), to(Wu), QQ, stream=stream)  # weight layout, once
    tau = torch.from_numpy((np.arange(M) % QQ).astype(np.int32)).to(dev)
    ws = Q.workspace(QQ, M, device=dev, dw_shape=(D, 2 * F))  # dW scratch for the training step
    H = torch.empty(M, F, dtype=torch.bfloat16, device=dev)
    Y = torch.empty(M, D, dtype=torch.bfloat16, device=dev)
    Q.qalg_build_index(tau, QQ, ws=ws, stream=stream)
    r = Q.QALG_FLAG_INDEX_READY
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    for _ in range(3):
        Q.qalg_gated_forward(Xd, Wgu, tau, QQ, H=H, ws=ws, flags=r, stream=stream)
        Q.qalg_forward(H, Wdd, tau, QQ, Y=Y, ws=ws, flags=r, stream=stream)
    torch.cuda.synchronize()
    n = 10
    a, b, cc = ev(), ev(), ev()
    tg = td = 0.0
    for _ in range(n):
        a.record(stream)
        Q.qalg_gated_forward(Xd, Wgu, tau, QQ, H=H, ws=ws, flags=r, stream=stream)
        b.record(stream)
        Q.qalg_forward(H, Wdd, tau, QQ, Y=Y, ws=ws, flags=r, stream=stream)
        cc.record(stream)
        torch.cuda.synchronize()
        tg += a.elapsed_time(b)
        td += b.elapsed_time(cc)
    tg, td = tg / n, td / n
    flop = 2.0 * rho(QQ) * M * D * F  # per projection (gate, up and down each)
    res = {"workload": "gated_ffn_D4096_F12288_q8_M16384_bf16", "gate_up_ms": round(tg, 4),
           "gate_up_tflops": round(2 * flop / (tg * 1e-3) / 1e12, 1), "down_ms": round(td, 4),
           "step_ms": round(tg + td, 4), "step_tflops": round(3 * flop / ((tg + td) * 1e-3) / 1e12, 1)}
    res["training"] = gated_train(Q, torch, np, synth, dev, stream, Xd, Wgu, Wdd, tau, ws, H, Y, flop)
    log(f"[bench] gated FFN leg: {res}")
    return res


def gated_train(Q, torch, np, synth, dev, stream, Xd, Wgu, Wdd, tau, ws, H, Y, flop):
    """Training step of the gated FFN on the merged layout: merged forward keeping the pre-activations
    with H computed in the same launch, down forward; down dX and dW, pointwise SwiGLU VJP, merged dX
    and dW.  9 projections (section 6.2)."""
    r = Q.QALG_FLAG_INDEX_READY
    dY = torch.from_numpy(synth.normal_operand(6005, (M, D), 1.0, "bf16").bits.view(np.int16)).view(
        torch.bfloat16).to(dev)
    GU = torch.empty(M, 2 * F, dtype=torch.bfloat16, device=dev)
    dGU = torch.empty_like(GU)
    dH = torch.empty(M, F, dtype=torch.bfloat16, device=dev)
    dX = torch.empty(M, D, dtype=torch.bfloat16, device=dev)
    dWd = torch.empty(F, D, dtype=torch.bfloat16, device=dev)
    dWgu = torch.empty(D, 2 * F, dtype=torch.bfloat16, device=dev)
    ops = [
        # gate/up products kept in bf16 for the VJP, and H from them, in one launch
        ("fwd_gate_up", lambda: Q.qalg_gated_forward_keep(Xd, Wgu, tau, QQ, H=H, GU=GU, ws=ws, flags=r,
                                                          stream=stream)),
        ("fwd_down", lambda: Q.qalg_forward(H, Wdd, tau, QQ, Y=Y, ws=ws, flags=r, stream=stream)),
        ("dx_down", lambda: Q.qalg_backward_dx(dY, Wdd, tau, QQ, dX=dH, ws=ws, flags=r, stream=stream)),
        ("dw_down", lambda: Q.qalg_backward_dw(H, dY, tau, QQ, dW=dWd, ws=ws, flags=r, stream=stream)),
        ("swiglu_bwd", lambda: Q.qalg_swiglu_backward(GU, dH, QQ, dGU=dGU, stream=stream)),
        ("dx_gate_up", lambda: Q.qalg_backward_dx(dGU, Wgu, tau, QQ, dX=dX, ws=ws, flags=r, stream=stream)),
        ("dw_gate_up", lambda: Q.qalg_backward_dw(Xd, dGU, tau, QQ, dW=dWgu, ws=ws, flags=r, stream=stream)),
    ]
    for _ in range(2):
        for _, f in ops:
            f()
    torch.cuda.synchronize()
    n = 5
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(ops) + 1)]
    tot = [0.0] * len(ops)
    for _ in range(n):
        ev[0].record(stream)
        for k, (_, f) in enumerate(ops):
            f()
            ev[k + 1].record(stream)
        torch.cuda.synchronize()
        for k in range(len(ops)):
            tot[k] += ev[k].elapsed_time(ev[k + 1])
    ms = {name: t / n for (name, _), t in zip(ops, tot)}
    step = sum(ms.values())
    out = {f"{k}_ms": round(v, 4) for k, v in ms.items()}
    out["step_ms"] = round(step, 4)
    out["step_tflops"] = round(9 * flop / (step * 1e-3) / 1e12, 1)  # 9 projection-shaped products
    out["swiglu_bwd_GBs"] = round(10.0 * M * F / (ms["swiglu_bwd"] * 1e-3) / 1e9, 1)  # gate, up, dH in; 2 out
    return out


def pilot_leg(Q, torch, np, synth, dev, stream):
    """The pretraining pilot's FFN law (appendix D): Q_2^(x)2 on a bias-free SwiGLU FFN, D = 768,
    F = 1536, one 40 x 1536-position batch (M = 61440), the interval schedule floor((p mod 768) / 192).
    Timed: fused gate/up + down forwards under the recursive law, under Q_4 and at q = 1 (dense)."""
    c, Mp, Dp, Fp, qp = 7, 61440, 768, 1536, 4
    to = lambda op: torch.from_numpy(op.bits.view(np.int16)).view(torch.bfloat16).to(dev)  # noqa: E731
    X = to(synth.normal_operand(1000 * c + 1, (Mp, Dp), 1.0, "bf16"))
    Wg = to(synth.normal_operand(1000 * c + 2, (Dp, Fp), Dp ** -0.5, "bf16"))
    Wu = to(synth.normal_operand(1000 * c + 3, (Dp, Fp), Dp ** -0.5, "bf16"))
    Wd = to(synth.normal_operand(1000 * c + 4, (Fp, Dp), Fp ** -0.5, "bf16"))
    pos = torch.from_numpy(synth.cyclic_positions(Mp, 1536)).to(dev)
    H = torch.empty(Mp, Fp, dtype=torch.bfloat16, device=dev)
    Y = torch.empty(Mp, Dp, dtype=torch.bfloat16, device=dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    out = {"workload": "pilot_swiglu_ffn_D768_F1536_M61440_interval", "M": Mp, "D": Dp, "F": Fp}
    for name, q, law, frac in (("tensor_q4", qp, Q.QALG_FLAG_LAW_TENSOR, 9 / 16), ("complete_q4", qp, 0, 7 / 16),
                               ("dense_q1", 1, 0, 1.0)):
        tau = Q.qalg_type_schedule(pos, q, Q.QALG_SCHEDULE_INTERVAL, 768 if q > 1 else 1, stream=stream)
        ws = Q.workspace(q, Mp, device=dev)
        Q.qalg_build_index(tau, q, ws=ws, stream=stream)
        Wgu = Q.qalg_merge_gate_up(Wg, Wu, q, stream=stream)
        fl = law | Q.QALG_FLAG_INDEX_READY
        step = lambda: (Q.qalg_gated_forward(X, Wgu, tau, q, H=H, ws=ws, flags=fl, stream=stream),  # noqa: E731
                        Q.qalg_forward(H, Wd, tau, q, Y=Y, ws=ws, flags=fl, stream=stream))
        for _ in range(3):
            step()
        torch.cuda.synchronize()
        n = 20
        a, b = ev(), ev()
        a.record(stream)
        for _ in range(n):
            step()
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / n
        flop = 3 * 2.0 * frac * Mp * Dp * Fp
        out[name] = {"step_ms": round(ms, 4), "algebra_tflops": round(flop / (ms * 1e-3) / 1e12, 1)}
    # the training step (merged forward, SwiGLU, down; down dX and dW, SwiGLU VJP, merged dX and dW)
    dY = to(synth.normal_operand(1000 * c + 5, (Mp, Dp), 1.0, "bf16"))
    GU = torch.empty(Mp, 2 * Fp, dtype=torch.bfloat16, device=dev)
    dGU = torch.empty_like(GU)
    dH = torch.empty(Mp, Fp, dtype=torch.bfloat16, device=dev)
    dX = torch.empty(Mp, Dp, dtype=torch.bfloat16, device=dev)
    dWd = torch.empty(Fp, Dp, dtype=torch.bfloat16, device=dev)
    dWgu = torch.empty(Dp, 2 * Fp, dtype=torch.bfloat16, device=dev)
    for name, q, law, frac in (("tensor_q4", qp, Q.QALG_FLAG_LAW_TENSOR, 9 / 16), ("complete_q4", qp, 0, 7 / 16),
                               ("dense_q1", 1, 0, 1.0)):
        tau = Q.qalg_type_schedule(pos, q, Q.QALG_SCHEDULE_INTERVAL, 768 if q > 1 else 1, stream=stream)
        # a workspace that lets dW split its contraction (the largest dW: D x 2F)
        ws = Q.workspace(q, Mp, device=dev, dw_shape=(Dp, 2 * Fp))
        Q.qalg_build_index(tau, q, ws=ws, stream=stream)
        Wgu = Q.qalg_merge_gate_up(Wg, Wu, q, stream=stream)
        fl = law | Q.QALG_FLAG_INDEX_READY

        def train():
            Q.qalg_gated_forward_keep(X, Wgu, tau, q, H=H, GU=GU, ws=ws, flags=fl, stream=stream)
            Q.qalg_forward(H, Wd, tau, q, Y=Y, ws=ws, flags=fl, stream=stream)
            Q.qalg_backward_dx(dY, Wd, tau, q, dX=dH, ws=ws, flags=fl, stream=stream)
            Q.qalg_backward_dw(H, dY, tau, q, dW=dWd, ws=ws, flags=fl, stream=stream)
            Q.qalg_swiglu_backward(GU, dH, q, dGU=dGU, stream=stream)
            Q.qalg_backward_dx(dGU, Wgu, tau, q, dX=dX, ws=ws, flags=fl, stream=stream)
            Q.qalg_backward_dw(X, dGU, tau, q, dW=dWgu, ws=ws, flags=fl, stream=stream)

        for _ in range(2):
            train()
        torch.cuda.synchronize()
        n = 10
        a, b = ev(), ev()
        a.record(stream)
        for _ in range(n):
            train()
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / n
        flop = 9 * 2.0 * frac * Mp * Dp * Fp
        out[name]["train_step_ms"] = round(ms, 4)
        out[name]["train_algebra_tflops"] = round(flop / (ms * 1e-3) / 1e12, 1)
    out["train_speedup_tensor_vs_dense"] = round(out["dense_q1"]["train_step_ms"] / out["tensor_q4"]["train_step_ms"], 3)
    out["speedup_tensor_vs_dense"] = round(out["dense_q1"]["step_ms"] / out["tensor_q4"]["step_ms"], 3)
    out["speedup_complete_vs_dense"] = round(out["dense_q1"]["step_ms"] / out["complete_q4"]["step_ms"], 3)
    log(f"[bench] pilot FFN leg: {out}")
    return out


def few_rows_leg(Q, torch, np, synth, dev, stream):
    """Few rows per type (appendix E's q = 32 projections at M = 2048, 64 rows per type): the
    Qwen3-8B and Qwen3-1.7B FFN shapes, up and down, at q = 32 and with the same kernels at q = 1."""
    c, Mf, q = 8, 2048, 32
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    out = {"workload": "q32_M2048_projections", "M": Mf, "q": q}
    for name, D, F in (("qwen3_8b", 4096, 12288), ("qwen3_1_7b", 2048, 6144)):
        for direction, K, N in (("up", D, F), ("down", F, D)):
            X = torch.from_numpy(synth.normal_operand(1000 * c + 1, (Mf, K), 1.0, "bf16").bits.view(np.int16)).view(
                torch.bfloat16).to(dev)
            W = torch.from_numpy(synth.normal_operand(1000 * c + 2, (K, N), K ** -0.5, "bf16").bits.view(
                np.int16)).view(torch.bfloat16).to(dev)
            Y = torch.empty(Mf, N, dtype=torch.bfloat16, device=dev)
            res = {}
            for qq in (q, 1):
                tau = torch.from_numpy((np.arange(Mf) % qq).astype(np.int32)).to(dev)
                ws = Q.workspace(qq, Mf, device=dev)
                Q.qalg_build_index(tau, qq, ws=ws, stream=stream)
                fl = Q.QALG_FLAG_INDEX_READY
                for _ in range(5):
                    Q.qalg_forward(X, W, tau, qq, Y=Y, ws=ws, flags=fl, stream=stream)
                torch.cuda.synchronize()
                n = 40
                a, b = ev(), ev()
                a.record(stream)
                for _ in range(n):
                    Q.qalg_forward(X, W, tau, qq, Y=Y, ws=ws, flags=fl, stream=stream)
                b.record(stream)
                torch.cuda.synchronize()
                res[qq] = a.elapsed_time(b) / n
            flop = 2.0 * rho(q) * Mf * K * N
            out[f"{name}_{direction}"] = {"K": K, "N": N, "q32_us": round(res[q] * 1e3, 1),
                                          "q32_algebra_tflops": round(flop / (res[q] * 1e-3) / 1e12, 1),
                                          "q1_us": round(res[1] * 1e3, 1),
                                          "speedup_vs_q1": round(res[1] / res[q], 2)}
    log(f"[bench] few-rows leg: {out}")
    return out


def attention_leg(Q, torch, np, synth, dev, stream):
    """Causal attention with the algebraic score (appendix G): 32 query heads, 8 key/value heads,
    d = 128, S = 4096 (one sequence), q = 4 under Q_4 and under Q_2^(x)2, and the same kernel at
    q = 1 (ordinary attention).  FLOP: 2 |F| m per allowed pair for QK^T plus 2 d for PV.
    Training (Algorithm 2 with step 9): the forward that keeps the log-sum-exp, then the gradients,
    which recompute the scores twice and form dQ and dK over the compared groups (4 score-sized
    products) and dP twice and dV (3 d-sized products per allowed pair)."""
    c, Hq, Hkv, S, d, q = 9, 32, 8, 4096, 128, 4
    to = lambda op: torch.from_numpy(op.bits.view(np.int16)).view(torch.bfloat16).to(dev)  # noqa: E731
    Qd = to(synth.normal_operand(1000 * c + 1, (Hq, S, d), 1.0, "bf16"))
    Kd = to(synth.normal_operand(1000 * c + 2, (Hkv, S, d), 1.0, "bf16"))
    Vd = to(synth.normal_operand(1000 * c + 3, (Hkv, S, d), 1.0, "bf16"))
    Od = torch.empty_like(Qd)
    dOd = to(synth.normal_operand(1000 * c + 4, (Hq, S, d), 1.0, "bf16"))
    lse = torch.empty((Hq, S), dtype=torch.float32, device=dev)
    dQd, dKd, dVd = torch.empty_like(Qd), torch.empty_like(Kd), torch.empty_like(Vd)
    ws_b = torch.empty(Q.qalg_attention_backward_workspace_bytes(Hq, Hkv, S, d, q), dtype=torch.uint8, device=dev)
    pairs = S * (S + 1) // 2
    same = {}  # allowed pairs with equal types, per q (cyclic types)
    for qq in (1, q):
        n = [(S - i + qq - 1) // qq for i in range(qq)]
        same[qq] = sum(k * (k + 1) // 2 for k in n)
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    out = {"workload": "causal_attention_Hq32_Hkv8_S4096_d128", "Hq": Hq, "Hkv": Hkv, "S": S, "d": d}
    for name, qq, fl in (("complete_q4", q, 0), ("tensor_q4", q, Q.QALG_FLAG_LAW_TENSOR), ("dense_q1", 1, 0)):
        run = lambda: Q.qalg_attention_forward(Qd, Kd, Vd, qq, O=Od, flags=fl, stream=stream)  # noqa: E731
        for _ in range(3):
            run()
        torch.cuda.synchronize()
        n = 10
        a, b = ev(), ev()
        a.record(stream)
        for _ in range(n):
            run()
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / n
        m = d // qq
        if fl:   # recursive law at L = 2: |F| = 2^popcount(i ^ j); mean over cyclic pairs, exact below
            score = 0
            for i in range(qq):
                for j in range(qq):
                    ni = (S - i + qq - 1) // qq
                    cnt = sum(max(0, (i + qq * t - j) // qq + 1) for t in range(ni))  # keys j + q t' <= i + q t
                    score += cnt * (1 << bin(i ^ j).count("1")) * m
        else:
            score = (2 * pairs - same[qq]) * m if qq > 1 else pairs * d
        flop = 2.0 * Hq * (score + pairs * d)
        out[name] = {"ms": round(ms, 4), "algebra_tflops": round(flop / (ms * 1e-3) / 1e12, 1),
                     "score_fraction": round(score / (pairs * d), 4)}
        # training: forward with lse, then the gradients
        fwd_t = lambda: Q.qalg_attention_forward_train(Qd, Kd, Vd, qq, 0, O=Od, lse=lse, flags=fl, stream=stream)  # noqa: E731
        bwd = lambda: Q.qalg_attention_backward(Qd, Kd, Vd, Od, dOd, lse, qq, 0, dQ=dQd, dK=dKd, dV=dVd, ws=ws_b,  # noqa: E731
                                                flags=fl, stream=stream)
        for _ in range(2):
            fwd_t()
            bwd()
        torch.cuda.synchronize()
        ts = [ev() for _ in range(2 * n + 1)]
        ts[0].record(stream)
        for k in range(n):
            fwd_t()
            ts[2 * k + 1].record(stream)
            bwd()
            ts[2 * k + 2].record(stream)
        torch.cuda.synchronize()
        f_ms = sum(ts[2 * k].elapsed_time(ts[2 * k + 1]) for k in range(n)) / n
        b_ms = sum(ts[2 * k + 1].elapsed_time(ts[2 * k + 2]) for k in range(n)) / n
        bflop = 2.0 * Hq * (4 * score + 3 * pairs * d)
        out[name].update({"train_fwd_ms": round(f_ms, 4), "bwd_ms": round(b_ms, 4),
                          "bwd_algebra_tflops": round(bflop / (b_ms * 1e-3) / 1e12, 1),
                          "train_step_ms": round(f_ms + b_ms, 4)})
    for name in ("complete_q4", "tensor_q4"):
        out[name]["speedup_vs_q1"] = round(out["dense_q1"]["ms"] / out[name]["ms"], 3)
        out[name]["train_speedup_vs_q1"] = round(out["dense_q1"]["train_step_ms"] / out[name]["train_step_ms"], 3)
        rho = out[name]["score_fraction"]
        out[name]["ceiling"] = round(2 / (1 + rho), 3)   # eq 46
    log(f"[bench] attention leg: {out}")
    return out


def attention_decode_leg(Q, torch, np, synth, dev, proto):
    """Cached decoding with the algebraic score (appendix G, Algorithm 3): 32 sequences, one new
    row each, 32 query heads over 8 key/value heads (GQA), d = 128, caches of 4096 slots where
    sequence b holds positions 0 .. 4095 - b (the rest empty), q = 4 and its q = 1 control (the
    same kernel, ordinary attention).  HBM-bound: the algorithmic bytes are each allowed slot's
    value row, the F(i, j) groups of its key row (eq 57: m or 2m of the d features), the slot
    positions, Q and O."""
    c, B, Hq, Hkv, N, d, q = 11, 32, 32, 8, 4096, 128, 4
    to = lambda op: torch.from_numpy(op.bits.view(np.int16)).view(torch.bfloat16).to(dev)  # noqa: E731
    Qn = to(synth.normal_operand(1000 * c + 1, (B, Hq, d), 1.0, "bf16"))
    Kc = to(synth.normal_operand(1000 * c + 2, (B, Hkv, N, d), 1.0, "bf16"))
    Vc = to(synth.normal_operand(1000 * c + 3, (B, Hkv, N, d), 1.0, "bf16"))
    lens = N - np.arange(B)
    key_pos = np.full((B, N), -1, np.int64)
    for b in range(B):
        key_pos[b, :lens[b]] = np.arange(lens[b])
    q_pos = (lens - 1).astype(np.int64)
    qp, kp = torch.from_numpy(q_pos).to(dev), torch.from_numpy(key_pos).to(dev)
    O = torch.empty(B, Hq, d, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(Q.qalg_attention_decode_workspace_bytes(B, Hq, N, d), dtype=torch.uint8, device=dev)
    res = {"workload": "attn_decode_B32_Hq32_Hkv8_N4096_d128_q4_bf16", "cache": "sequence b: positions 0..4095-b"}
    per_q = {}
    for qq in (q, 1):
        m = d // qq
        kbytes = 0
        for b in range(B):
            i = int(q_pos[b]) % qq
            js = np.arange(lens[b]) % qq
            kbytes += int(np.where(js == i, m, 2 * m).sum()) * 2 * Hkv
        vbytes = int(lens.sum()) * d * 2 * Hkv
        per_q[qq] = kbytes + vbytes + B * N * 8 + 2 * B * Hq * d * 2
    g_q = proto.capture(lambda st: Q.qalg_attention_decode(Qn, Kc, Vc, qp, kp, q, O=O, ws=ws, stream=st))
    g_1 = proto.capture(lambda st: Q.qalg_attention_decode(Qn, Kc, Vc, qp, kp, 1, O=O, ws=ws, stream=st))
    cmp_ = proto.compare(g_q, g_1)
    for key, t, t1 in (("warm", cmp_["warm"]["median_ms"], cmp_["warm_q1"]["median_ms"]),
                       ("flushed", cmp_["flushed_ms"], cmp_["flushed_q1_ms"])):
        cmp_[f"{key}_GBs"] = round(per_q[q] / (t * 1e-3) / 1e9, 1)
        cmp_[f"{key}_frac_hbm"] = round(per_q[q] / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
        cmp_[f"{key}_q1_GBs"] = round(per_q[1] / (t1 * 1e-3) / 1e9, 1)
    cmp_["algorithmic_bytes"] = per_q[q]
    cmp_["algorithmic_bytes_q1"] = per_q[1]
    cmp_["byte_ratio_q1_over_q"] = round(per_q[1] / per_q[q], 3)   # the ceiling the byte cut allows
    res.update(cmp_)
    log(f"[bench] attention decode leg: {res}")
    return res


def decode_leg(Q, torch, np, synth, dev, stream):
    """64 experts, one token row each (KV-cached decode), (7168 -> 2048) q = 4, weight-streaming path."""
    c = 4
    E, K, N, q, Mx = 64, 7168, 2048, 4, 1
    Wb = np.stack([synth.normal_operand(1000 * c + 100 + e, (K, N), K ** -0.5, "bf16").bits for e in range(E)])
    Xb = np.stack([synth.normal_operand(1000 * c + 300 + e, (Mx, K), 1.0, "bf16").bits for e in range(E)])
    pos = np.stack([synth.random_positions(1000 * c + 200 + e, Mx) for e in range(E)])
    taus = (pos % q).astype(np.int32)
    to = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)  # noqa: E731
    W, X = to(Wb), to(Xb)
    tau = torch.from_numpy(taus).to(dev)
    Y = torch.empty(E, Mx, N, dtype=torch.bfloat16, device=dev)
    ws = Q.workspace(q, Mx, E, device=dev)
    fn = lambda: Q.qalg_forward_batched(X, W, tau, q, Y=Y, ws=ws, stream=stream)  # noqa: E731
    s, r = K // q, N // q
    # algorithmic bytes: every weight block some row needs, once, plus X and Y
    wbytes = 0
    for e in range(E):
        present = set(int(t) for t in taus[e])
        nblocks = q + sum(q - 1 for _ in present)  # all W_jj plus the strip W_i, off-diagonal, per present type
        wbytes += nblocks * s * r * 2
    byts = wbytes + E * Mx * (K + N) * 2
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    times = []
    for k in range(12):
        # evict L2 and the MALL between single launches: write the buffer, then
        # read it back, so that the caches hold clean lines of it and the
        # write-back of its dirty lines does not land inside the timed launch
        flush.fill_(k & 0xFF)
        flush.view(torch.float32).sum()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    ms = float(np.median(times[2:]))
    res = {"workload": "decode_64experts_7168x2048_q4_M1_bf16", "ms": round(ms, 4),
           "algorithmic_bytes": byts, "GBs": round(byts / (ms * 1e-3) / 1e9, 1),
           "frac_hbm": round(byts / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4), "protocol": "flushed (1 GiB written, then read)"}
    log(f"[bench] decode leg: {res}")
    return res


def experts_leg(Q, torch, np, synth, dev, stream):
    """Narrow MoE expert shapes (section 7.1's expert projections): 64 experts, each with its own
    bank, M in {1, 8, 64, 256, 1024} tokens per expert at random absolute positions (tau = p mod q),
    (7168 -> 2048, q = 4), (2048 -> 768, q = 4 and q = 8).  Each launch is timed alone after a
    1 GiB cache flush (the 64 banks of 2048 x 768 would otherwise sit in the MALL), against the
    same kernels at q = 1.  X and positions of M rows are the first M rows of the 1024-row draws
    (the seeded streams are prefix-consistent), as in the parity test of this workload."""
    c, E, MS = 4, 64, (1, 8, 64, 256, 1024)
    to = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)  # noqa: E731
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)

    def flushed(fn, reps=8):
        times = []
        for k in range(reps + 2):
            flush.fill_(k & 0xFF)
            flush.view(torch.float32).sum()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        return float(np.median(times[2:]))

    res = {"workload": "experts_64_bf16", "protocol": "flushed (1 GiB written, then read), median of 8"}
    pos_all = np.stack([synth.random_positions(1000 * c + 200 + e, MS[-1]) for e in range(E)])
    for K, N in ((7168, 2048), (2048, 768)):
        with ThreadPoolExecutor(max_workers=8) as ex:
            Wb = list(ex.map(lambda e: synth.normal_operand(1000 * c + 100 + e, (K, N), K ** -0.5, "bf16").bits,
                             range(E)))
            Xb = list(ex.map(lambda e: synth.normal_operand(1000 * c + 300 + e, (MS[-1], K), 1.0, "bf16").bits,
                             range(E)))
        W = to(np.stack(Wb))
        X_all = to(np.stack(Xb))
        del Wb, Xb
        for q in ((4,) if K == 7168 else (4, 8)):
            s, r = K // q, N // q
            for Mx in MS:
                X = X_all[:, :Mx].contiguous()
                taus = (pos_all[:, :Mx] % q).astype(np.int32)
                tau = torch.from_numpy(taus).to(dev)
                tau1 = torch.zeros_like(tau)
                Y = torch.empty(E, Mx, N, dtype=torch.bfloat16, device=dev)
                ws, ws1 = Q.workspace(q, Mx, E, device=dev), Q.workspace(1, Mx, E, device=dev)
                t_q = flushed(lambda: Q.qalg_forward_batched(X, W, tau, q, Y=Y, ws=ws, stream=stream))
                t_1 = flushed(lambda: Q.qalg_forward_batched(X, W, tau1, 1, Y=Y, ws=ws1, stream=stream))
                t_2s = t_mk = None
                if Mx >= 8:
                    # section 5.3's second schedule (diagonal maps over all rows, then the strips)
                    ws2 = Q.workspace(q, Mx, E, device=dev, two_stage_N=N)
                    t_2s = flushed(lambda: Q.qalg_forward_batched(X, W, tau, q, Y=Y, ws=ws2, stream=stream,
                                                                  flags=Q.QALG_FLAG_TWO_STAGE))
                    del ws2
                    t_mk = flushed(lambda: Q.qalg_forward_batched(X, W, tau, q, Y=Y, ws=ws, stream=stream,
                                                                  flags=Q.QALG_FLAG_MASKED))
                flop = 2.0 * rho(q) * E * Mx * K * N
                wblocks = sum(q + (q - 1) * len(set(int(t) for t in taus[e])) for e in range(E))
                byts = wblocks * s * r * 2 + E * Mx * (K + N) * 2
                res[f"{K}x{N}_q{q}_M{Mx}"] = {
                    "ms": round(t_q, 4), "q1_ms": round(t_1, 4), "speedup_vs_q1": round(t_1 / t_q, 3),
                    "two_stage_ms": round(t_2s, 4) if t_2s else None,
                    "two_stage_speedup_vs_q1": round(t_1 / t_2s, 3) if t_2s else None,
                    "masked_ms": round(t_mk, 4) if t_mk else None,
                    "masked_speedup_vs_q1": round(t_1 / t_mk, 3) if t_mk else None,
                    "algebra_tflops": round(flop / (t_q * 1e-3) / 1e12, 1),
                    "GBs": round(byts / (t_q * 1e-3) / 1e9, 1)}
        del W, X_all
    log(f"[bench] experts leg: {res}")
    return res


def cpu_leg(np, host, rows, threads=None):
    """The fp64 oracle (NumPy/OpenBLAS) on the first `rows` rows of both projections, on all host
    cores (threads=None) or on `threads` BLAS threads."""
    import contextlib
    from oracle import qalg_oracle as O
    try:
        import threadpoolctl
        limit = threadpoolctl.threadpool_limits(limits=threads, user_api="blas") if threads else contextlib.nullcontext()
    except Exception:  # pragma: no cover - informational only
        threadpoolctl, limit = None, contextlib.nullcontext()
    rows = min(rows, M)
    tau = (np.arange(rows) % QQ).astype(np.int32)
    Xu = host["Xu"].f64[:rows]
    Xd = host["Xd"].f64[:rows]
    Wu = host["Wu"].f64
    Wd = host["Wd"].f64
    with limit:
        used = 0
        if threadpoolctl is not None:
            info = threadpoolctl.threadpool_info()
            used = max([i.get("num_threads", 0) for i in info if i.get("user_api") == "blas"] or [0])
        t0 = time.perf_counter()
        O.row_typed_forward(Xu, Wu, tau, QQ)
        O.row_typed_forward(Xd, Wd, tau, QQ)
        dt = time.perf_counter() - t0
    threads = used
    flop = 2 * 2.0 * rho(QQ) * rows * D * F
    res = {"value": round(flop / dt / 1e12, 5), "unit": "TFLOP/s", "cores": threads or len(os.sched_getaffinity(0)),
           "kind": "oracle", "seconds": round(dt, 2),
           "sample": f"first {rows} of {M} rows of the up and down projections (fp64 NumPy/OpenBLAS)"}
    log(f"[bench] cpu oracle: {res}")
    return res


if __name__ == "__main__":
    sys.exit(main())
