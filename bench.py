#!/usr/bin/env python3
"""Throughput of the batched verify-window MoE layer on one MI355X.

A step is one verify window through the whole layer: router GEMV + softmax + top-k +
per-expert row grouping, fused dequant gate/up + SwiGLU, down and the weighted combine with
the shared expert. By default one strata_window_layer call per window (router GEMV, then
gate/up whose workgroups take the routing themselves, then down and combine); --path split
runs strata_window_route and then strata_window_moe instead. The default
workload is the 8-row window (4 slots x token + MTP proposal, Zipf(1.1) router prior,
correlated pairs) of a 2048-hidden / 768-ffn / 128-expert top-8 layer with 4-bit block
quantization. --workload stack24_head runs the 24-layer stack with the 8-bit head instead (a step is
then one window through all 24 layers and the head).

Timing: K steps are captured into one HIP graph (inputs resident in HBM) and replayed
once between two synchronisations; steps cycle through L independent layer instances so
that the 256 MB Infinity Cache cannot serve a layer's weights from a previous visit.
The achieved bandwidth counts the unique weight bytes each window reads (router +
(distinct routed experts + 1 shared) x expert bytes), from the window's own routing.

Prints one JSON line.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E peak, 8 TB/s
METRIC = "verify-window MoE layer rows/s and achieved HBM GB/s (% of peak), 1 GPU"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2048)
    p.add_argument("--warmup", type=int, default=32)
    p.add_argument("--workload", default="four_slots_mtp_zipf",
                   choices=["two_slots_mtp", "four_slots_mtp_zipf", "stack24_head", "e256_2bit"])
    p.add_argument("--rows", type=int, default=None, help="window rows (e256_2bit row sweep)")
    p.add_argument("--layers", type=int, default=16, help="layer instances to cycle through")
    p.add_argument("--windows", type=int, default=256, help="distinct activation windows")
    p.add_argument("--prof-steps", type=int, default=512, help="eager steps timed per kernel")
    p.add_argument("--inflight", type=int, default=1,
                   help="independent windows in flight (windows alternate over this many streams, "
                        "like pipelined slot groups); 1 = one window after the other")
    p.add_argument("--path", choices=["layer", "split", "stack"], default=None,
                   help="layer (the default for one layer): strata_window_layer (router, then gate/up with "
                        "the routing in every workgroup, then down); split: strata_window_route, then "
                        "strata_window_moe; stack (the default for stack24_head): the whole stack and the "
                        "head in one strata_window_stack call")
    p.add_argument("--cpu-seconds", type=float, default=20.0,
                   help="oracle sample budget on all host threads (0: skip); a quarter of it more on one thread")
    p.add_argument("--replays", type=int, default=20,
                   help="further replays of the timed graph, whose median is reported beside the timed one")
    p.add_argument("--calibrate-copy-mib", type=int, default=0,
                   help="first copy this many MiB device to device three times (a dispatch of known "
                        "bytes for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    return p.parse_args()


def calibration_copy(torch, mib):
    """Three plain device-to-device copies of mib MiB (torch's copy kernel)."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] calibration copy: 3 x {mib} MiB read + {mib} MiB written")
    del src, dst


def stream_read_gbs(torch, sw, gib=2, reps=10):
    """The bandwidth a plain streaming read of HBM reaches on this GPU
    (strata_window_stream_read over gib GiB, the mean of reps dispatches, each timed by
    events that the dispatch records)."""
    src = torch.ones(gib << 28, dtype=torch.int32, device="cuda")   # gib GiB
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    for _ in range(2):
        sw.strata_window_stream_read(src, sink)
    evs = events(torch, 2 * reps)
    for i in range(reps):
        sw.strata_window_stream_read(src, sink, prof=[evs[2 * i].cuda_event, evs[2 * i + 1].cuda_event])
    torch.cuda.synchronize()
    ms = sum(evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(reps)) / reps
    nbytes = src.numel() * 4
    del src, sink
    return nbytes / (ms * 1e-3) / 1e9


def replay_median_ms(torch, g, n):
    """Median duration of n further replays of graph g (each between two events)."""
    out = []
    for _ in range(n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1))
    out.sort()
    return out[len(out) // 2]


def bpw(bits):
    """Bytes per weight including the per-block metadata (4 bytes per 32 weights)."""
    return bits / 8.0 + 4.0 / 32.0


def code_text(path):
    """A C++ source's code: comments removed, each line stripped, blank lines dropped (so a
    comment edit leaves the kernel's fingerprint, and its counter summary, valid)."""
    s = open(path, encoding="utf-8").read()
    s = re.sub(r"/\*.*?\*/", " ", s, flags=re.S)
    s = re.sub(r"//[^\n]*", "", s)
    return "\n".join(ln.strip() for ln in s.split("\n") if ln.strip())


def source_sha(files):
    """sha256 (first 16 hex digits) of the files' code text, in order."""
    h = hashlib.sha256()
    for f in files:
        h.update(code_text(os.path.join(ROOT, f)).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]


KERNEL_SOURCES = ["verify_window_expert_amd/csrc/moe.hip", "verify_window_expert_amd/csrc/common.h",
                  "verify_window_expert_amd/csrc/route_core.h"]


def counter_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary, when it was taken from the
    current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and line.startswith("- "):
            k, v = line[2:].split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("source_sha256_16") != source_sha(KERNEL_SOURCES):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def route_views(sw, torch, n, R, E, k):
    """n sets of routing outputs, as views into padded device arrays (16-byte aligned
    slices): (the arrays by name, the n RouteOut views)."""
    A = min(E, R * k) + 1
    ent = R * k + R
    pad = lambda m: (m + 63) // 64 * 64
    i32, f32 = torch.int32, torch.float32
    dev = "cuda"
    big = dict(topk_idx=torch.empty(n, pad(R * k), dtype=i32, device=dev),
               topk_w=torch.empty(n, pad(R * k), dtype=f32, device=dev),
               n_active=torch.zeros(n, 64, dtype=i32, device=dev),
               active=torch.empty(n, pad(A), dtype=i32, device=dev),
               offsets=torch.empty(n, pad(A + 1), dtype=i32, device=dev),
               entry_row=torch.empty(n, pad(ent), dtype=i32, device=dev),
               entry_w=torch.empty(n, pad(ent), dtype=f32, device=dev),
               row_mask=torch.empty(n, pad(E + 1), dtype=torch.uint8, device=dev),
               entry_pos=torch.empty(n, pad(ent), dtype=i32, device=dev),
               row_w=torch.empty(n, pad(R * (k + 1)), dtype=f32, device=dev))
    views = []
    for i in range(n):
        ro = sw.RouteOut.__new__(sw.RouteOut)
        ro.rows, ro.n_experts, ro.top_k = R, E, k
        for name, t in big.items():
            setattr(ro, name, t[i])
        views.append(ro)
    return big, views


class Steps:
    """Device state of K steps: layers, windows, per-step routing outputs, workspaces."""

    def __init__(self, cfg, n_layers, n_windows, steps, sw, torch, synth, DevLayer, to_dev_x, inflight=1,
                 path="layer", out_per_step=False, keep_host_layers=False):
        self.cfg, self.sw, self.torch = cfg, sw, torch
        self.path = path
        R, H, E, k = cfg.rows, cfg.hidden, cfg.experts, cfg.top_k
        t0 = time.time()
        self.layers = []
        self.host_layers = []
        self.host_layer0 = None
        for l in range(n_layers):
            L = synth.make_layer(cfg, l)
            self.layers.append(DevLayer(L, cfg))
            if l == 0:
                self.host_layer0 = L
            if keep_host_layers:
                self.host_layers.append(L)
            log(f"[bench] layer {l + 1}/{n_layers} resident ({time.time() - t0:.1f}s)")
        self.xs = [to_dev_x(synth.make_window(cfg, w, rows=R)) for w in range(n_windows)]
        # per-step routing outputs (so the timed graph holds no copies)
        dev = "cuda"
        self.big, self.routes = route_views(sw, torch, steps, R, E, k)
        # one set of workspaces and outputs per window in flight
        self.ws_r = [sw.workspace(sw.workspace_bytes(0, R, H, n_experts=E)) for _ in range(inflight)]
        self.ws_m = [sw.workspace(sw.workspace_bytes(1 if path == "split" else 3, R, H, cfg.ffn, E, k))
                     for _ in range(inflight)]
        # one output per window in flight (each step its own with out_per_step)
        self.out = [torch.empty(R, H, dtype=torch.float32, device=dev)
                    for _ in range(steps if out_per_step else inflight)]
        self.out_per_step = out_per_step
        self.inflight = inflight

    def step(self, i, prof=None):
        """One window; prof: None or 6 event handles (router start/end, gate/up start/end,
        down start/end)."""
        cfg, sw = self.cfg, self.sw
        dl = self.layers[i % len(self.layers)]
        x = self.xs[i % len(self.xs)]
        j = i % self.inflight
        out = self.out[i if self.out_per_step else j]
        if self.path == "layer":
            sw.strata_window_layer(x, dl.gate_w, dl.bias, cfg.top_k, dl.gate, dl.up, dl.down, *dl.sh,
                                   route=self.routes[i], out=out, ws=self.ws_m[j], prof=prof)
            return
        ro = sw.strata_window_route(x, dl.gate_w, dl.bias, cfg.top_k, out=self.routes[i], ws=self.ws_r[j],
                                    prof=None if prof is None else prof[:2])
        sw.strata_window_moe(x, dl.gate, dl.up, dl.down, *dl.sh, ro, out=out, ws=self.ws_m[j],
                             prof=None if prof is None else prof[2:])

    def layer_calls(self, steps, evs):
        """The C arguments of strata_window_layer for steps 0 .. steps-1, marshalled once,
        each step's dispatches recording 6 of evs (router start/end, gate/up start/end,
        down start/end of the combine): calling them back to back keeps the host ahead of
        the GPU, so that the recorded kernels run as they do in the timed graph."""
        import ctypes
        sw, cfg = self.sw, self.cfg
        L = sw.library()
        stream = ctypes.c_void_p(self.torch.cuda.current_stream().cuda_stream)
        keep, calls = [], []
        for i in range(steps):
            dl = self.layers[i % len(self.layers)]
            x = self.xs[i % len(self.xs)]
            j = i % self.inflight
            out = self.out[i if self.out_per_step else j]
            qs = [q.c() for q in (dl.gate, dl.up, dl.down, *dl.sh)]
            ro = self.routes[i].c()
            ev = (ctypes.c_void_p * 6)(*[e.cuda_event for e in evs[6 * i: 6 * i + 6]])
            ws = self.ws_m[j]
            args = (stream, ctypes.c_void_p(x.data_ptr()), 0 if x.dtype == self.torch.float32 else 1, cfg.rows,
                    cfg.hidden, cfg.ffn, ctypes.c_void_p(dl.gate_w.data_ptr()),
                    None if dl.bias is None else ctypes.c_void_p(dl.bias.data_ptr()), 0,
                    *[ctypes.byref(q) for q in qs], cfg.experts, cfg.top_k, ctypes.byref(ro), None,
                    ctypes.c_void_p(out.data_ptr()), None, ctypes.c_void_p(ws.data_ptr()),
                    ws.numel() * ws.element_size(), ev)
            keep.append((qs, ro, ev))
            calls.append(args)
        fn = L.strata_window_layer

        def run():
            for a in calls:
                rc = fn(*a)
                if rc:
                    raise RuntimeError(L.strata_window_last_error().decode())
        run.keep = keep
        return run

    def distinct_experts(self, steps):
        return (self.big["n_active"][:steps, 0] - 1).cpu().numpy()


def capture_steps(torch, st, K, NF=1):
    """One HIP graph of steps 0 .. K-1 of st: window i on stream i % NF (one stream: the
    windows run one after the other), every launch of the window's kernels in it."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    side = [torch.cuda.Stream() for _ in range(NF - 1)]
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for t in side:
                t.wait_stream(s)
            lanes = [s] + side
            for i in range(K):
                with torch.cuda.stream(lanes[i % NF]):
                    st.step(i)
            for t in side:
                s.wait_stream(t)
    torch.cuda.synchronize()
    return g


def device_layer_types(torch, sw):
    """Upload helpers: a layer's weights and a window's activations on the device."""
    import numpy as np

    def to_dev_x(x):
        if x.dtype == np.float32:
            return torch.from_numpy(np.ascontiguousarray(x)).cuda()
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)

    class DevLayer:
        def __init__(self, layer, cfg):
            H, F, b = cfg.hidden, cfg.ffn, cfg.bits
            self.gate_w = torch.from_numpy(layer.gate_w).cuda()
            self.bias = None if layer.bias is None else torch.from_numpy(layer.bias).cuda()
            up = lambda m, r, c: sw.upload_qmat(m[0], m[1], r, c, b)
            self.gate, self.up, self.down = up(layer.gate, F, H), up(layer.up, F, H), up(layer.down, H, F)
            self.sh = (up(layer.sh_gate, F, H), up(layer.sh_up, F, H), up(layer.sh_down, H, F))

    return DevLayer, to_dev_x


def events(torch, n):
    """n timing events, created (recorded once) so their handles exist."""
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    return evs


def window_tail_kernels(torch, sw, st, cfg, P):
    """Average durations (us, events recorded by the dispatches) of the window's small
    steps after the layer: the sampled draw of the window's rows from vocabulary-151936
    logits (N(0, 3^2), temperature 0.8, top_k 64, top_p 0.95, min_p 0.02), the greedy
    verify/accept of the slots' proposals (rows as token/proposal pairs, argmax and
    proposals synthetic) and the routing counts of the adaptive tier (count-only windows
    and selection rounds), from the steps' routing."""
    R, E = cfg.rows, cfg.experts
    g = torch.Generator(device="cpu").manual_seed(7)
    V = 151936
    logits = (torch.randn(R, V, generator=g) * 3).cuda()
    sparams = sw.sample_params([(0.8, 64, 0.95, 0.02, 1000 + r // 2) for r in range(R)])
    spos = torch.arange(R, dtype=torch.int64).cuda()
    sws = sw.workspace(sw.workspace_bytes(5, R, 0, vocab=V))
    stok = sw.strata_window_sample(logits, sparams, spos, ws=sws)
    argmax = torch.randint(0, V, (R,), generator=g, dtype=torch.int32).cuda()
    mtp = R % 2 == 0                        # token/proposal pairs; one row per slot otherwise
    prop = argmax[0::2].clone()
    prop[1::2] += 1                         # half the proposals kept
    counts = torch.zeros(E, dtype=torch.float32, device="cuda")
    resident = (torch.arange(E) % 3 == 0).to(torch.uint8).cuda()
    tok, ntok, nacc = sw.strata_window_accept(argmax, prop, mtp=mtp)
    out = {}
    for name, fn in (("sample", lambda i, ev: sw.strata_window_sample(logits, sparams, spos, tokens=stok, ws=sws,
                                                                      prof=ev)),
                     ("accept", lambda i, ev: sw.strata_window_accept(argmax, prop, mtp=mtp, tokens=tok,
                                                                      n_tokens=ntok, n_accepted=nacc, prof=ev)),
                     ("tier_count", lambda i, ev: sw.strata_window_tier(st.routes[i].row_mask, counts, 0.875,
                                                                        prof=ev)),
                     ("tier_select", lambda i, ev: sw.strata_window_tier(st.routes[i].row_mask, counts, 0.875,
                                                                         resident, 8, 1.5, prof=ev))):
        evs = events(torch, 2 * P)
        for i in range(P):
            fn(i, [evs[2 * i].cuda_event, evs[2 * i + 1].cuda_event])
        torch.cuda.synchronize()
        out[name] = round(1e3 * sum(evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(P)) / P, 3)
    return out


def cpu_baseline(cfg, host_layer, seconds, threads=None):
    """The CPU oracle, as it stands, on windows of the same workload until `seconds` pass
    (on `threads` OpenMP threads, else all the host offers)."""
    import oracle
    import synth
    oracle.build(force=False)
    all_threads = oracle.threads()
    if threads:
        oracle.set_threads(threads)
    H, F, E, b = cfg.hidden, cfg.ffn, cfg.experts, cfg.bits
    q = lambda m, n, r, c: oracle.qmat(m[0], m[1], r, c, b, n)
    L = host_layer
    mats = (q(L.gate, E, F, H), q(L.up, E, F, H), q(L.down, E, H, F),
            q(L.sh_gate, 1, F, H), q(L.sh_up, 1, F, H), q(L.sh_down, 1, H, F))
    n, t0 = 0, time.time()
    while True:
        x = synth.make_window(cfg, n, rows=cfg.rows)
        _, _, idx, w = oracle.route(x, L.gate_w, L.bias, cfg.top_k)
        oracle.group(idx, w, E)
        oracle.moe(x, *mats, idx, w)
        n += 1
        if time.time() - t0 >= seconds:
            break
    dt = time.time() - t0
    used = oracle.threads()
    oracle.set_threads(all_threads)
    return {"value": round(cfg.rows * n / dt, 3), "unit": "rows/s", "cores": used, "kind": "oracle",
            "sample": f"{n} windows of this workload (layer instance 0, windows 0..{n - 1}): route, grouping and "
                      f"experts, {dt:.1f} s wall clock, OpenMP threads = {used}"}


def cpu_baseline_stack(cfg, seconds, threads=None):
    """The CPU oracle on the stack workload, sampled: whole layers of the stack (window 0's
    rows through layers 0, 1, ... with the residual, each layer's input the previous one's
    x_next) until about 3/4 of `seconds` pass, then the head on a slice of the vocabulary
    for the rest; one window's time = 24 x the mean layer time + the head time scaled to
    the whole vocabulary."""
    import oracle
    import synth
    oracle.build(force=False)
    all_threads = oracle.threads()
    if threads:
        oracle.set_threads(threads)
    H, F, E, b, K = cfg.hidden, cfg.ffn, cfg.experts, cfg.bits, cfg.top_k
    q = lambda m, n, r, c: oracle.qmat(m[0], m[1], r, c, b, n)
    x = synth.make_window(cfg, 0)
    n, t_layers, t0 = 0, 0.0, time.time()
    while n < cfg.layers:
        L = synth.make_layer(cfg, n)
        mats = (q(L.gate, E, F, H), q(L.up, E, F, H), q(L.down, E, H, F),
                q(L.sh_gate, 1, F, H), q(L.sh_up, 1, F, H), q(L.sh_down, 1, H, F))
        t1 = time.time()
        _, _, idx, w = oracle.route(x, L.gate_w, L.bias, K)
        oracle.group(idx, w, E)
        _, x = oracle.moe(x, *mats, idx, w, residual=x, want_x_next=True)
        t_layers += time.time() - t1
        n += 1
        if time.time() - t0 >= 0.75 * seconds:
            break
    codes, meta = synth.make_head(cfg)
    hq = oracle.qmat(codes[0], meta[0], cfg.vocab, H, 8)
    v1, t_head = 1024, 0.0
    while True:
        t1 = time.time()
        oracle.head(x, hq, 0, v1)
        t_head = time.time() - t1
        if time.time() - t0 >= seconds or v1 >= cfg.vocab:
            break
        v1 = min(cfg.vocab, v1 * 2)
    window_s = cfg.layers * t_layers / n + t_head * cfg.vocab / v1
    used = oracle.threads()
    oracle.set_threads(all_threads)
    return {"value": round(cfg.rows / window_s, 4), "unit": "rows/s", "cores": used, "kind": "oracle",
            "sample": f"window 0 through layers 0..{n - 1} of the stack ({t_layers / n:.2f} s per layer) and the head "
                      f"on vocabulary entries 0..{v1 - 1} ({t_head:.2f} s); one window = {cfg.layers} layers + the "
                      f"whole head, scaled: {window_s:.1f} s; OpenMP threads = {used}"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the window is measured on one GPU: the path has no multi-GPU mode (--gpus must be 1)"}))
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(2)
    import synth
    import verify_window_expert_amd as sw
    sw.library()   # raises if the HIP library is not built
    DevLayer, to_dev_x = device_layer_types(torch, sw)
    if args.calibrate_copy_mib > 0:
        calibration_copy(torch, args.calibrate_copy_mib)

    if args.workload == "stack24_head":
        args.path = args.path or "stack"
        return bench_stack(args, torch, synth, sw, DevLayer, to_dev_x)
    args.path = args.path or "layer"
    if args.path == "stack":
        print(json.dumps({"error": "--path stack is for --workload stack24_head"}))
        sys.exit(2)
    cfg = synth.config(args.workload, **({"rows": args.rows} if args.rows else {}))
    K, W = args.steps, args.warmup
    NF = max(1, args.inflight)
    st = Steps(cfg, args.layers, args.windows, max(K, args.prof_steps), sw, torch, synth, DevLayer, to_dev_x, NF,
               args.path)

    for i in range(W):
        st.step(i)
    torch.cuda.synchronize()

    # ---- per-kernel durations: eager steps, events recorded by the dispatches themselves
    P = min(args.prof_steps, K)
    evs = events(torch, 6 * P)
    if args.path == "layer":
        run = st.layer_calls(P, evs)   # marshalled once: the host stays ahead of the GPU
        run()                          # warm
        torch.cuda.synchronize()
        run()
    else:
        for i in range(P):
            e = evs[6 * i: 6 * i + 6]
            st.step(i, prof=[ev.cuda_event for ev in e])
    torch.cuda.synchronize()
    # the eager steps' own pace: first router start to last combine end, per window
    eager_ms_per_step = evs[0].elapsed_time(evs[6 * (P - 1) + 5]) / P
    d_route = [evs[6 * i].elapsed_time(evs[6 * i + 1]) for i in range(P)]
    d_gu = [evs[6 * i + 2].elapsed_time(evs[6 * i + 3]) for i in range(P)]
    d_dn = [evs[6 * i + 4].elapsed_time(evs[6 * i + 5]) for i in range(P)]
    U_prof = st.distinct_experts(P)
    d_post = window_tail_kernels(torch, sw, st, cfg, P)

    # ---- the timed region: one graph of K steps (window i on stream i % inflight; the
    # windows of one stream run one after the other)
    g = capture_steps(torch, st, K, NF)
    g.replay()                      # warm replay
    torch.cuda.synchronize()
    # replay() runs on the current stream: the events go there too
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = e0.elapsed_time(e1)
    ms_med = replay_median_ms(torch, g, args.replays) if args.replays > 0 else None
    U = st.distinct_experts(K)

    H, F, E, R = cfg.hidden, cfg.ffn, cfg.experts, cfg.rows
    b_x = 3 * F * H * bpw(cfg.bits)
    b_r = 4 * E * H + (4 * E if cfg.zipf else 0)
    bytes_total = float(sum(b_r + (u + 1) * b_x for u in U))
    gbs = bytes_total / (ms_total * 1e-3) / 1e9
    rows_s = R * K / (ms_total * 1e-3)

    # dominant kernel: gate/up (two thirds of the window's bytes)
    gu_bytes = [(u + 1) * 2 * F * H * bpw(cfg.bits) for u in U_prof]
    gu_gbs = sum(gu_bytes) / (sum(d_gu) * 1e-3) / 1e9
    traffic = counter_traffic("k_gateup", cfg.name)
    roof = {"bound": "hbm", "achieved": round(gu_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gu_gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
            "kernel": ("k_gateup (fused {}-bit dequant gate/up matvec + SwiGLU{})".format(
                cfg.bits, ", with the window's top-k and grouping in every workgroup" if args.path == "layer" else "")),
            "avg_launch_us": round(1e3 * sum(d_gu) / P, 3),
            "algorithmic_bytes_per_launch": round(sum(gu_bytes) / P)}

    del g
    torch.cuda.synchronize()
    log("[bench] streaming read of 2 GiB")
    stream = stream_read_gbs(torch, sw)
    cpu = cpu1 = None
    if args.cpu_seconds > 0:
        log(f"[bench] CPU oracle sample ({args.cpu_seconds:.0f} s budget, then a quarter of it on one thread)")
        cpu = cpu_baseline(cfg, st.host_layer0, args.cpu_seconds)
        cpu1 = cpu_baseline(cfg, st.host_layer0, args.cpu_seconds / 4, threads=1)

    workload = {"four_slots_mtp_zipf": "one MoE layer, 8-row verify window (4 slots x token+MTP proposal, Zipf(1.1) router prior, "
                   "correlated pairs), hidden 2048, ffn 768, 128 experts top-8 + shared, 4-bit blocks of 32",
                "two_slots_mtp": "one MoE layer, 4-row verify window (2 slots with MTP), hidden 2048, ffn 768, 128 experts top-8 "
                   "+ shared, 4-bit blocks of 32",
                "e256_2bit": f"one MoE layer, {R}-row window, hidden 4096, ffn 1024, 256 experts top-8 + shared, 2-bit "
                   "blocks of 32"}[cfg.name]
    line = {
        "metric": METRIC, "value": round(rows_s, 1), "unit": "rows/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms_total / K, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": workload, "name": cfg.name, "rows": R, "hidden": H, "ffn": F, "experts": E,
                   "top_k": cfg.top_k, "bits": cfg.bits, "layer_instances": args.layers,
                   "windows_in_flight": NF, "path": args.path},
        "hbm_gbs": round(gbs, 1), "hbm_frac_of_peak": round(gbs / PEAK_HBM_GBS, 4),
        "stream_read_gbs": round(stream, 1), "hbm_frac_of_stream_read": round(gbs / stream, 4),
        "ms_per_step_median_of_replays": None if ms_med is None else round(ms_med / K, 5),
        "replays": args.replays,
        "mean_distinct_experts": round(float(U.mean()), 2),
        "unique_weight_bytes_per_window": round(bytes_total / K),
        "kernel_us": dict({"route": round(1e3 * sum(d_route) / P, 3), "gateup": round(1e3 * sum(d_gu) / P, 3),
                           "down": round(1e3 * sum(d_dn) / P, 3)}, **d_post),
        "kernel_us_source": ("dispatch-recorded events of {} eager windows issued back to back from arguments "
                             "marshalled once (the host ahead of the GPU, as in the graph)".format(P)
                             if args.path == "layer" else "dispatch-recorded events of {} eager windows".format(P)),
        "eager_ms_per_step": round(eager_ms_per_step, 5),
        "wall_s": round(wall, 4),
        "roofline": roof, "cpu_baseline": cpu, "cpu_baseline_1_thread": cpu1,
    }
    print(json.dumps(line), flush=True)


def bench_stack(args, torch, synth, sw, DevLayer, to_dev_x):
    """24 layers + head per step (the layer-stack workload)."""
    cfg = synth.config("stack24_head")
    K, W = min(args.steps, 256), min(args.warmup, 8)
    R, H, F, E, k = cfg.rows, cfg.hidden, cfg.ffn, cfg.experts, cfg.top_k
    t0 = time.time()
    layers = []
    for l in range(cfg.layers):
        layers.append(DevLayer(synth.make_layer(cfg, l), cfg))
        log(f"[bench] layer {l + 1}/{cfg.layers} resident ({time.time() - t0:.1f}s)")
    codes, meta = synth.make_head(cfg)
    head = sw.upload_qmat(codes, meta, cfg.vocab, H, 8)
    xs = [to_dev_x(synth.make_window(cfg, w)) for w in range(16)]
    # per-step, per-layer routing outputs: the timed graph holds the stack's kernels only
    big, rviews = route_views(sw, torch, K * cfg.layers, R, E, k)
    routes_of = lambda i: rviews[(i % K) * cfg.layers:(i % K + 1) * cfg.layers]
    ws_r = sw.workspace(sw.workspace_bytes(0, R, H, n_experts=E))
    ws_m = sw.workspace(sw.workspace_bytes(1 if args.path == "split" else 3, R, H, F, E, k))
    ws_h = sw.workspace(sw.workspace_bytes(2, R, H, vocab=cfg.vocab))
    xa = torch.empty(R, H, dtype=torch.bfloat16, device="cuda")
    xb = torch.empty_like(xa)
    out = torch.empty(R, H, dtype=torch.float32, device="cuda")
    logits = torch.empty(R, cfg.vocab, dtype=torch.float32, device="cuda")
    am = torch.empty(8, dtype=torch.int32, device="cuda")
    stack_layers = [(dl.gate_w, dl.bias, dl.gate, dl.up, dl.down, *dl.sh) for dl in layers]
    ws_s = sw.workspace(sw.workspace_bytes(4, R, H, F, E, k, cfg.vocab)) if args.path == "stack" else None

    def step(i, prof_head=None):
        x0, routes = xs[i % len(xs)], routes_of(i)
        if args.path == "stack":
            sw.strata_window_stack(x0, stack_layers, k, head=head, routes=routes, logits=logits, argmax=am, out=out,
                                   x_final=xb, ws=ws_s)
            if prof_head is not None:   # the head's own duration: the same head once more, timed
                sw.strata_window_head(xb, head, logits=logits, argmax=am, ws=ws_h, prof=prof_head)
            return
        # layer 0 reads the window itself; the later inputs alternate between xa and xb
        cur, nxt = x0, xa
        for l, dl in enumerate(layers):
            if args.path == "layer":
                sw.strata_window_layer(cur, dl.gate_w, dl.bias, k, dl.gate, dl.up, dl.down, *dl.sh,
                                       route=routes[l], residual=cur, out=out, x_next=nxt, ws=ws_m)
            else:
                ro = sw.strata_window_route(cur, dl.gate_w, dl.bias, k, out=routes[l], ws=ws_r)
                sw.strata_window_moe(cur, dl.gate, dl.up, dl.down, *dl.sh, ro, residual=cur, out=out, x_next=nxt,
                                     ws=ws_m)
            cur, nxt = nxt, (xb if nxt is xa else xa)
        sw.strata_window_head(cur, head, logits=logits, argmax=am, ws=ws_h, prof=prof_head)

    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    # the head's duration: events recorded by its own dispatches, over eager steps
    P = 16
    hev = events(torch, 2 * P)
    for i in range(P):
        step(i, prof_head=[hev[2 * i].cuda_event, hev[2 * i + 1].cuda_event])
    torch.cuda.synchronize()
    head_us = 1e3 * sum(hev[2 * i].elapsed_time(hev[2 * i + 1]) for i in range(P)) / P
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(K):
                step(i)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    ms_med = replay_median_ms(torch, g, min(args.replays, 5)) if args.replays > 0 else None
    # every step's routing, as the replays wrote it: [step][layer] distinct routed experts
    U = (big["n_active"][:K * cfg.layers, 0].view(K, cfg.layers) - 1).cpu().numpy()
    b_x = 3 * F * H * bpw(cfg.bits)
    b_h = cfg.vocab * H * (1 + 2 / 32)
    bytes_total = float((4 * E * H + (U + 1) * b_x).sum() + K * b_h)
    gbs = bytes_total / (ms * 1e-3) / 1e9
    line = {"metric": METRIC, "value": round(R * K / (ms * 1e-3), 1), "unit": "rows/s", "n_gpus": 1, "steps": K,
            "warmup": W, "ms_per_step": round(ms / K, 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "24 MoE layers (hidden 2048, ffn 768, 128 experts top-8 + shared, 4-bit) with "
                                   "residual, then an 8-bit head of vocab 151936 with argmax, 8-row window",
                       "name": "stack24_head", "path": args.path},
            "hbm_gbs": round(gbs, 1), "hbm_frac_of_peak": round(gbs / PEAK_HBM_GBS, 4),
            "ms_per_step_median_of_replays": None if ms_med is None else round(ms_med / K, 5),
            "kernel_us": {"head": round(head_us, 3)},
            "roofline": {"bound": "hbm", "achieved": round(b_h / (head_us * 1e-6) / 1e9, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(b_h / (head_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                         "traffic": None, "kernel": "k_head + k_head_argmax (8-bit head GEMV, vocab 151936)",
                         "avg_launch_us": round(head_us, 3), "algorithmic_bytes_per_launch": round(b_h)},
            "cpu_baseline": None}
    if args.cpu_seconds > 0:
        log(f"[bench] CPU oracle sample ({args.cpu_seconds:.0f} s budget)")
        line["cpu_baseline"] = cpu_baseline_stack(cfg, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
