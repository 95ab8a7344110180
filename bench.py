#!/usr/bin/env python3
"""Throughput of the routed MoE FFN layer on one MI355X.

One step = one pass of the whole layer (router GEMM, top-k routing, grouping by
expert, grouped gate/up SwiGLU GEMM with the shared expert, grouped down GEMM,
weighted combine) over one batch, through the C-ABI entry moe_layer_forward.
Inputs are seeded synthetic tensors drawn on the GPU and resident in HBM before
the timed region.  The primary line is the 512-token decode batch (D=4096,
512 experts of I=1024, top-10, one shared expert of I=1024, bf16).  The same
run also measures ("secondary") the 8192-token prefill chunk of that layer, the
skewed-popularity prefill, one GPU's fp8 expert-parallel share (64 of 512
experts, routing given) and the tiny fp32 layer.

Prints ONE JSON line.  `roofline` is for the dominant kernel (the grouped
gate/up GEMM), timed live with HIP events recorded on the launch stream around
it in every timed step; `measured_peaks` is the streaming-read bandwidth of a
plain read kernel on the same device; `cpu_baseline` times the CPU oracle on
the host cores.
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

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # dense bf16 MFMA
FP8_PEAK_TFLOPS = 5000.0     # dense fp8 MFMA
METRIC = "MoE-layer tokens/sec on 1 MI355X (T=512 decode, T=8192 prefill) + % roofline"
_ES = {"f32": 4, "bf16": 2, "e4m3": 1}


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="decode_bf16")
    p.add_argument("--layout", default="packed", choices=["packed", "rows"],
                   help="expert weight layout (packed: repacked once by moe_pack_weights before timing)")
    p.add_argument("--secondary",
                   default="prefill_bf16,skew_prefill_bf16,prefill32k_bf16,decode_fp8,ep_share_fp8,tiny_fp32",
                   help="comma-separated workloads also measured ('' for none); the bf16 ones reuse the weights")
    p.add_argument("--secondary-steps", type=int, default=50)
    p.add_argument("--no-hbm-probe", action="store_true", help="skip the streaming-read bandwidth probe")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-tokens", type=int, default=0, help="tokens of the oracle sample (0: whole batch)")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="also run a plain device copy of this many MiB (calibrates HBM counters)")
    return p.parse_args()


def code_tokens(text):
    """C++ source without comments and with each run of whitespace as one space (string and character
    literals kept as they are), so that editing a comment leaves the result unchanged."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash():
    """Hash of the code the grouped GEMM kernel is built from, comments excluded (its traffic figures are void
    once the code changes)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_moe_ffn_route_amd", "csrc")
    for f in ("common.hpp", "gemm.hpp", "gemm.hip"):
        h.update(code_tokens(open(os.path.join(csrc, f)).read()).encode())
    return h.hexdigest()[:16]


def committed_traffic(workload):
    """HBM bytes per gate/up launch from the committed counter summary, if it matches these kernels."""
    path = os.path.join(ROOT, "profiles", f"gemm_gate_up_{workload}_pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"kernel_source_hash:\s*`?([0-9a-f]+)", text)
    m_val = re.search(r"traffic_bytes_per_launch:\s*`?([0-9.eE+]+)", text)
    if not m_src or not m_val or m_src.group(1) != kernel_source_hash():
        return None
    return float(m_val.group(1))


class Layer:
    """Buffers and launch of one workload (device inputs shared with another workload when given)."""

    def __init__(self, wl, inp, packed_w=None):
        import torch
        import sparse_moe_ffn_route_amd as moe
        self.torch, self.moe, self.wl, self.inp = torch, moe, wl, inp
        self.dims = moe.make_dims(wl.T, wl.D, wl.E, wl.top_k, wl.I, wl.I_shared, wl.expert_begin, wl.local,
                                  wl.renormalize, wl.act, wl.w, wl.out, "packed" if packed_w else "rows")
        pw = packed_w or {n: getattr(inp, n) for n in ("w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")}
        self.ws = moe.workspace(self.dims)
        out_dt = torch.float32 if wl.out == "f32" else torch.bfloat16
        self.y = torch.empty(wl.T, wl.D, dtype=out_dt, device="cuda")
        self.logits = None if wl.routing_given else torch.empty(wl.T, wl.E, dtype=torch.float32, device="cuda")
        self.packed = torch.empty(wl.T, 2, wl.top_k, dtype=torch.int32, device="cuda")
        sh = wl.I_shared > 0
        self.pw = pw
        self.weights = moe.make_weights(inp.w_router, pw["w_gate"], pw["w_up"], pw["w_down"], inp.s_gate, inp.s_up,
                                        inp.s_down, pw["ws_gate"] if sh else None, pw["ws_up"] if sh else None,
                                        pw["ws_down"] if sh else None)

    def step(self, events=None):
        self.moe.moe_layer_forward(self.dims, self.weights, self.inp.x, self.inp.packed, self.inp.bias, self.y,
                                   self.logits, self.packed, self.ws, stage_events=events)

    def new_events(self):
        evs = [self.torch.cuda.Event(enable_timing=True) for _ in range(self.moe.STAGE_EVENTS)]
        for e in evs:
            e.record()       # torch creates the underlying hipEvent on first record
        return evs

    def run(self, steps, warmup):
        torch = self.torch
        for _ in range(warmup):
            self.step()
        ev_sets = [self.new_events() for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(ev_sets[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        stages = {name: [] for name in self.moe.STAGES}
        self.step_ms = []
        for evs in ev_sets:
            for j, name in enumerate(self.moe.STAGES):
                stages[name].append(evs[j].elapsed_time(evs[j + 1]))
            self.step_ms.append(evs[0].elapsed_time(evs[-1]))
        return wall, {k: sum(v) / len(v) for k, v in stages.items()}

    # ---- algorithmic work ---------------------------------------------------
    def routing_stats(self):
        torch = self.torch
        ids = self.packed[:, 0, :].reshape(-1).long() - self.wl.expert_begin
        ids = ids[(ids >= 0) & (ids < self.wl.local)]
        counts = torch.bincount(ids, minlength=self.wl.local)
        return int(ids.numel()), int((counts > 0).sum().item()), counts

    def work(self):
        wl = self.wl
        n_a, active, counts = self.routing_stats()
        wb, ab = _ES[wl.w], _ES[wl.act]
        hb = 4 if wl.act == "f32" else 2
        ob = _ES[wl.out]
        scales = (2 * wl.I + wl.D) * 4 if wl.w == "e4m3" else 0
        expert_w = active * (3 * wl.D * wl.I * wb + scales)
        shared_w = 3 * wl.D * wl.I_shared * ab
        router_w = 0 if wl.routing_given else wl.E * wl.D * ab
        io = wl.T * wl.D * ab + wl.T * wl.D * ob + wl.T * 2 * wl.top_k * 4
        layer_bytes = expert_w + shared_w + router_w + io
        layer_flop = (0 if wl.routing_given else 2 * wl.T * wl.D * wl.E) + n_a * 6 * wl.D * wl.I \
            + wl.T * 6 * wl.D * wl.I_shared
        # routed gate/up kernel: gate+up weights (and fp8 scales) of every active expert,
        # the gathered tokens' rows of x read once, h written once
        x_rows = int((self.packed[:, 0, :].long() - wl.expert_begin).ge(0).logical_and(
            (self.packed[:, 0, :].long() - wl.expert_begin).lt(wl.local)).any(dim=1).sum().item())
        xb = 1 if wl.w == "e4m3" else ab  # fp8 experts read the e4m3 copy of x (and a scale per row)
        gu_bytes = active * (2 * wl.D * wl.I * wb + (2 * wl.I * 4 if wl.w == "e4m3" else 0)) \
            + x_rows * (wl.D * xb + (4 if wl.w == "e4m3" else 0)) + n_a * wl.I * hb
        gu_flop = n_a * 4 * wl.D * wl.I
        return dict(n_assign=n_a, active_experts=active, max_rows=int(counts.max().item()),
                    layer_bytes=layer_bytes, layer_flop=layer_flop, gate_up_bytes=gu_bytes, gate_up_flop=gu_flop)


def layer_summary(layer, wall, stages, steps):
    wl = layer.wl
    w = layer.work()
    ms = wall / steps * 1e3
    peak_tf = FP8_PEAK_TFLOPS if wl.w == "e4m3" else BF16_PEAK_TFLOPS
    hbm_frac = w["layer_bytes"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS
    mfma_frac = w["layer_flop"] / (ms * 1e-3) / 1e12 / peak_tf
    q = sorted(layer.step_ms)
    pick = lambda f: round(q[min(len(q) - 1, int(f * (len(q) - 1) + 0.5))], 4)
    return dict(workload=wl.name, tokens_per_s=wl.T / (ms * 1e-3), ms_per_step=ms,
                step_ms_events={"p10": pick(0.1), "median": pick(0.5), "p90": pick(0.9), "n": len(q)},
                layer_hbm_frac=hbm_frac, layer_mfma_frac=mfma_frac,
                layer_roofline_frac=max(hbm_frac, mfma_frac), stage_ms=stages, work=w)


def roofline_of(layer, stages, summary=None):
    w = layer.work()
    t = stages["gate_up"] * 1e-3
    achieved = w["gate_up_bytes"] / t / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": committed_traffic(layer.wl.name),
            "layer_frac": None if summary is None else round(summary["layer_roofline_frac"], 4),
            "kernel": f"gemm_kernel<{layer.wl.w},SwiGLU> (routed grouped gate/up)",
            "bytes_per_launch": w["gate_up_bytes"], "avg_launch_ms": round(stages["gate_up"], 4),
            "mfma_TFLOPs": round(w["gate_up_flop"] / t / 1e12, 1)}


def cpu_baseline(layer, sample_tokens):
    """The oracle, as it stands, on the host cores: routing from the GPU's fp32 logits, then the layer."""
    import numpy as np
    import threadpoolctl
    import torch
    import oracle
    import synth
    wl, inp = layer.wl, layer.inp
    T = wl.T if sample_tokens <= 0 else min(sample_tokens, wl.T)
    cores = len(os.sched_getaffinity(0))
    # host copies of the stored inputs (not timed)
    host = synth.LayerInputs(wl, inp.x[:T].cpu(), None, inp.w_gate.cpu(), inp.w_up.cpu(), inp.w_down.cpu(),
                             None if inp.s_gate is None else inp.s_gate.cpu(),
                             None if inp.s_up is None else inp.s_up.cpu(),
                             None if inp.s_down is None else inp.s_down.cpu(),
                             None if inp.ws_gate is None else inp.ws_gate.cpu(),
                             None if inp.ws_up is None else inp.ws_up.cpu(),
                             None if inp.ws_down is None else inp.ws_down.cpu())
    logits = None if layer.logits is None else layer.logits[:T].cpu().numpy()
    packed = layer.packed[:T].cpu().numpy()
    bias = None if inp.bias is None else inp.bias.cpu().numpy()
    x64 = synth.f64(host.x)
    torch.set_num_threads(cores)
    with threadpoolctl.threadpool_limits(cores):
        t0 = time.perf_counter()
        if wl.routing_given:
            ids, w32 = oracle.unpack_routing(packed)
            w = w32.astype(np.float64)
        else:
            ids, w = oracle.route(logits, wl.top_k, bias=bias, renormalize=wl.renormalize)
        if wl.w == "e4m3":
            oracle.layer_from_routing_fp8(x64, ids, w, synth.ExpertViewFP8(host), expert_begin=wl.expert_begin,
                                          n_local=wl.local)
        else:
            oracle.layer_from_routing(x64, ids, w, synth.ExpertView(host), shared=synth.shared_f64(host),
                                      expert_begin=wl.expert_begin, n_local=wl.local)
        dt = time.perf_counter() - t0
    return {"value": round(T / dt, 3), "unit": "tokens/s", "cores": cores, "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"first {T} tokens of the {wl.name} batch (T={wl.T}): fp64 NumPy oracle, routing from the "
                      f"GPU's fp32 logits, grouped experts, combine; {dt:.1f} s",
            "seconds": round(dt, 2)}


def copy_probe(mib):
    """A plain device-to-device copy of known size, for scaling the HBM byte counters."""
    import torch
    n = mib * 2 ** 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    return {"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}


def audit_of(layer, n_sample=16):
    """moe_audit of the last step's output on n_sample evenly spaced tokens: fp32 shadow vs the layer."""
    import torch
    import sparse_moe_ffn_route_amd as moe
    T = layer.wl.T
    sample = torch.linspace(0, T - 1, n_sample, device="cuda").to(torch.int32)
    layer.step()                                  # y and the routing blob of one call
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    res = moe.moe_audit(layer.dims, layer.weights, layer.inp.x, layer.inp.packed if layer.wl.routing_given
                        else layer.packed, layer.y, sample)
    e1.record()
    torch.cuda.synchronize()
    r = res.cpu().tolist()
    return {"samples": n_sample, "max_abs_err": r[0], "max_abs_ref": r[1], "rel_err": r[0] / r[1] if r[1] else None,
            "ms": round(e0.elapsed_time(e1), 3)}


def router_variants(wl, x, w_router, reps=20):
    """moe_route (projection GEMM + route kernel) against moe_route_fused on the same x, in microseconds."""
    import torch
    import sparse_moe_ffn_route_amd as moe
    T = x.shape[0]
    d = moe.make_dims(T, wl.D, wl.E, wl.top_k, wl.I, wl.I_shared, 0, wl.E, wl.renormalize, wl.act, wl.w, wl.out)
    ws = moe.workspace(d)
    logits = torch.empty(T, wl.E, dtype=torch.float32, device="cuda")
    packed = torch.empty(T, 2, wl.top_k, dtype=torch.int32, device="cuda")
    calls = {"two_kernel_us": lambda: moe.moe_route(d, x, w_router, logits, None, packed, ws=ws),
             "fused_us": lambda: moe.moe_route_fused(d, x, w_router, None, None, packed, ws=ws)}
    out = {}
    for name, fn in calls.items():
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        out[name] = round(e0.elapsed_time(e1) / reps * 1e3, 1)
    return out


def hbm_probe(buf, reps=5):
    """Best-of-reps streaming-read bandwidth (GB/s) of moe_hbm_read_probe over buf."""
    import torch
    import sparse_moe_ffn_route_amd as moe
    nbytes = buf.numel() * buf.element_size()
    nbytes -= nbytes % 16
    sink = torch.empty(moe.HBM_PROBE_SINK_WORDS, dtype=torch.int32, device="cuda")
    best = 0.0
    for _ in range(reps + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        moe.moe_hbm_read_probe(buf, sink)
        e1.record()
        torch.cuda.synchronize()
        best = max(best, nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    return round(best, 1)


def mfma_probe(dtype, iters=4000, reps=3):
    """Best-of-reps dense MFMA rate (TFLOP/s) of moe_mfma_peak_probe: register-only MFMA chains on every CU."""
    import torch
    import sparse_moe_ffn_route_amd as moe
    sink = torch.empty(moe.MFMA_PROBE_BLOCKS, dtype=torch.float32, device="cuda")
    best = 0.0
    for _ in range(reps + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        _, flop = moe.moe_mfma_peak_probe(dtype, iters, sink)
        e1.record()
        torch.cuda.synchronize()
        best = max(best, flop / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    return round(best, 1)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this layer is built and measured on one GPU; --gpus must be 1 "
                                   "(expert-parallel sharding across GPUs is a design note, not a run mode)"}))
        return 2

    import torch
    import synth
    torch.cuda.set_device(0)

    wl = synth.WORKLOADS[args.workload]
    t_gen = time.perf_counter()
    inp = synth.make_inputs(wl, seed=0, device="cuda")
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen
    print(f"[bench] inputs for {wl.name} drawn on the GPU in {t_gen:.1f} s", file=sys.stderr, flush=True)

    packed_w = None
    if args.layout == "packed":
        import sparse_moe_ffn_route_amd as moe
        packed_w = {n: (None if getattr(inp, n) is None else moe.moe_pack_weights(getattr(inp, n)))
                    for n in ("w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")}
        torch.cuda.synchronize()
    layer = Layer(wl, inp, packed_w)
    wall, stages = layer.run(args.steps, args.warmup)
    prim = layer_summary(layer, wall, stages, args.steps)
    print(f"[bench] {wl.name}: {prim['ms_per_step']:.3f} ms/step, stages {stages}", file=sys.stderr, flush=True)

    secondary = []
    for name in [n for n in args.secondary.split(",") if n]:
        wl2 = synth.WORKLOADS[name]
        same_layer = all(getattr(wl2, f) == getattr(wl, f) for f in ("D", "E", "I", "I_shared", "w", "act"))
        if same_layer and not wl2.routing_given:
            # same weights; new hidden states of the batch size (and the workload's logit bias)
            g = torch.Generator(device="cuda")
            g.manual_seed(synth._torch_seed(0, "x", 1))
            x2 = (torch.randn(wl2.T, wl2.D, generator=g, device="cuda")).to(torch.bfloat16)
            bias = None
            if wl2.skew_alpha is not None:
                bias = torch.from_numpy(synth.zipf_bias(wl2.E, wl2.skew_alpha, wl2.skew_s, wl2.skew_empty, 1)).cuda()
            inp2 = synth.LayerInputs(wl2, x2, inp.w_router, inp.w_gate, inp.w_up, inp.w_down, inp.s_gate, inp.s_up,
                                     inp.s_down, inp.ws_gate, inp.ws_up, inp.ws_down, bias, None)
            pw2 = packed_w
        else:
            inp2 = synth.make_inputs(wl2, seed=0, device="cuda")
            pw2 = None
            if args.layout == "packed":
                import sparse_moe_ffn_route_amd as moe
                pw2 = {n: (None if getattr(inp2, n) is None else moe.moe_pack_weights(getattr(inp2, n)))
                       for n in ("w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")}
        layer2 = Layer(wl2, inp2, pw2)
        wall2, stages2 = layer2.run(args.secondary_steps, 2)
        sec = layer_summary(layer2, wall2, stages2, args.secondary_steps)
        sec["roofline"] = roofline_of(layer2, stages2, sec)
        if wl2.w == "e4m3":
            sec["audit"] = audit_of(layer2)
        secondary.append(sec)
        print(f"[bench] {wl2.name}: {sec['ms_per_step']:.3f} ms/step, stages {stages2}", file=sys.stderr, flush=True)
        del layer2, inp2, pw2
        torch.cuda.empty_cache()

    routers = None
    if wl.E <= 512 and not wl.routing_given:
        g = torch.Generator(device="cuda")
        g.manual_seed(synth._torch_seed(0, "x", 1))
        x8k = (torch.randn(8192, wl.D, generator=g, device="cuda")).to(torch.bfloat16)
        routers = {f"T={inp.x.shape[0]}": router_variants(wl, inp.x, inp.w_router),
                   "T=8192": router_variants(wl, x8k, inp.w_router)}
        del x8k
        print(f"[bench] router variants: {routers}", file=sys.stderr, flush=True)

    measured = None
    if not args.no_hbm_probe:
        measured = {"hbm_read_GBs": hbm_probe(packed_w["w_gate"] if packed_w else inp.w_gate),
                    "how": "moe_hbm_read_probe over the expert gate weights (non-temporal 16-byte loads), best of 5",
                    "mfma_bf16_TFLOPs": mfma_probe("bf16"), "mfma_fp8_TFLOPs": mfma_probe("e4m3"),
                    "mfma_how": "moe_mfma_peak_probe: 2048 workgroups x 4 waves x 8 independent MFMA chains on "
                                "register operands (bf16 16x16x32, e4m3 16x16x128), best of 3"}
        print(f"[bench] streaming read: {measured['hbm_read_GBs']} GB/s, MFMA bf16 {measured['mfma_bf16_TFLOPs']} "
              f"fp8 {measured['mfma_fp8_TFLOPs']} TFLOP/s", file=sys.stderr, flush=True)

    probe = copy_probe(args.copy_probe_mib) if args.copy_probe_mib else None

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle ...", file=sys.stderr, flush=True)
        cpu = cpu_baseline(layer, args.cpu_sample_tokens)
        print(f"[bench] oracle: {cpu['seconds']} s", file=sys.stderr, flush=True)

    out = {
        "metric": METRIC,
        "value": round(prim["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(prim["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.w if wl.w == "e4m3" else wl.act,
        "data": "synthetic (seeded Philox draws on the GPU; random-init weights)",
        "config": {"workload": wl.name, "T": wl.T, "D": wl.D, "E": wl.E, "top_k": wl.top_k, "I": wl.I,
                   "I_shared": wl.I_shared, "expert_slice": [wl.expert_begin, wl.local],
                   "weight_layout": args.layout, "parallelism": "1 GPU"},
        "roofline": roofline_of(layer, stages, prim),
        "cpu_baseline": cpu,
        "layer": {k: prim[k] for k in ("layer_hbm_frac", "layer_mfma_frac", "layer_roofline_frac", "stage_ms",
                                        "step_ms_events")},
        "work": prim["work"],
        "secondary": secondary,
        "kernel_source_hash": kernel_source_hash(),
    }
    out["audit"] = audit_of(layer)
    if routers:
        out["router_variants"] = routers
    if measured:
        out["measured_peaks"] = measured
        out["roofline"]["frac_of_measured_hbm"] = round(out["roofline"]["achieved"] / measured["hbm_read_GBs"], 4)
        for sec in secondary:
            sec["roofline"]["frac_of_measured_hbm"] = round(sec["roofline"]["achieved"] / measured["hbm_read_GBs"], 4)
            peak = measured["mfma_fp8_TFLOPs"] if sec["workload"].endswith("fp8") else measured["mfma_bf16_TFLOPs"]
            sec["roofline"]["mfma_frac_of_measured"] = round(sec["roofline"]["mfma_TFLOPs"] / peak, 4)
    if probe:
        out["copy_probe"] = probe
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
