"""Decode-step throughput of the FSQ latent-decode path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one decode step of a whole model: for each layer, the new token's
residual state is appended (E projection, FSQ, packing) and the query attends
over the packed cache, both through one fsq_decode_step call (--two-call:
fsq_append + fsq_decode_attn, the same kernels plus one launch). Inputs are seeded
synthetic tensors of the workload's shapes, resident in HBM before timing.
Each step is replayed from a HIP graph; steps rotate over enough replicas of
the per-layer buffers that one step's data is never still in the 256 MB
Infinity Cache from its previous use.

Prints one JSON line: context-tokens/s (sum of sequence lengths / step time),
the step's roofline fraction, the split-K kernel's roofline (HIP events from
hipExtLaunchKernelGGL around each launch, in a second phase of eager steps), the
prefill append of the G=84 workload (8192 tokens through E and FSQ) with its
roofline, and the fp64 CPU oracle timed on a bounded sample of the same workload
(all threads and one thread), whose outputs are also compared with the GPU's.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, vendor figure
MFMA_FP16_PEAK_TFLOPS = 2500.0
MALL_BYTES = 256 * 2 ** 20
COMPARED = ("qwen3_8b_g256", "qwen3_8b_g84")   # workloads of the SDPA and key-reconstruction comparisons
# workloads whose line carries the oracle's CPU baseline and in-run parity
CPU_BASELINE_WORKLOADS = ("qwen3_8b_g256", "qwen3_8b_g84", "qwen3_1p7b_ragged", "qwen3_8b_g84_1m")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="qwen3_8b_g256", choices=sorted(synth.WORKLOADS))
    ap.add_argument("--also", default="qwen3_8b_g84,qwen3_1p7b_ragged,qwen3_8b_g84_1m,qwen3_8b_g32,"
                                      "qwen3_8b_g20,qwen3_8b_l4_g168,qwen3_8b_l256_g42",
                    help="comma-separated extra workloads reported under 'also' ('' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sdpa", action="store_true",
                    help="skip the PyTorch SDPA comparison on materialised K/V")
    ap.add_argument("--no-recon", action="store_true",
                    help="skip the key-reconstruction comparison")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-launch-floor", action="store_true",
                    help="skip timing the step's launch chain of trivial kernels")
    ap.add_argument("--no-layer-batched", action="store_true",
                    help="skip the layer-batched measurement (all layers' attention in one call)")
    ap.add_argument("--eager", action="store_true", help="launch without HIP graphs")
    ap.add_argument("--timing-steps", type=int, default=5,
                    help="eager steps whose split-K launches are bracketed by HIP events")
    ap.add_argument("--no-append", action="store_true", help="skip the prefill-append measurement")
    ap.add_argument("--append-only", action="store_true",
                    help="only the prefill-append measurement (with --eager: 12 eager calls)")
    ap.add_argument("--two-call", action="store_true",
                    help="per layer fsq_append + fsq_decode_attn instead of fsq_decode_step")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a device copy of this size (counter calibration) and exit")
    return ap.parse_args()


# ---------------------------------------------------------------- arithmetic
def decode_call_bytes(w, lens):
    codes = int(np.sum(lens)) * w.P
    wkv = 2 * w.n_kv * w.d_h * w.G * 2
    qo = 2 * w.batch * w.n_q * w.d_h * 2 + 4 * w.batch
    return codes + wkv + qo


def append_call_bytes(w):
    return w.G * w.C * 2 + w.batch * w.C * 2 + w.batch * w.P


def step_flops(w, lens):
    T = float(np.sum(lens))
    lat = 4.0 * w.n_q * w.G * T                       # scores + pooling
    per_seq = 4.0 * w.n_q * w.d_h * w.G * w.batch     # absorb + W_v
    app = 2.0 * w.batch * w.G * w.C
    return w.layers * (lat + per_seq + app)


# --------------------------------------------------------------- GPU side
class Model:
    """Per-layer device buffers of one replica of the workload."""

    def __init__(self, w, torch, replicas, on_chunk=None):
        import fsq_latent_decode_amd as fsq
        self.fsq, self.torch, self.w = fsq, torch, w
        dev = "cuda"
        self.lens_np = synth.seq_lens(w)
        self.cap = w.context
        self.lens = torch.from_numpy(self.lens_np).to(dev)

        def bf(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

        fsq_codes = self.fsq_cache(w, torch, bf, on_chunk) if w.codes_from_fsq else None
        base = []
        for l in range(w.layers):
            E, W = synth.layer_weights(w, l)
            if fsq_codes is not None:
                codes = fsq_codes.clone()
            else:
                codes = torch.from_numpy(synth.layer_codes(w, l, lens=self.lens_np if w.ragged else None)).to(dev)
            base.append(dict(E=bf(E), W=bf(W), q=bf(synth.layer_query(w, l)),
                             x=bf(synth.layer_x(w, l, w.batch, synth.T_XNEW)), codes=codes))
        del fsq_codes
        self.reps = [base]
        for _ in range(replicas - 1):
            self.reps.append([{k: v.clone() for k, v in d.items()} for d in base])
        for rep in self.reps:
            for d in rep:
                d["out"] = torch.empty((w.batch, w.n_q, w.d_h), dtype=torch.bfloat16, device=dev)
        self.ws = fsq.alloc_workspace(w.batch, w.n_q, w.G, self.cap, dev)
        torch.cuda.synchronize()

    def fsq_cache(self, w, torch, bf, on_chunk=None, chunk=8192):
        """A cache whose codes are FSQ(E x) (the million-token workload): layer
        0's prefill chunks appended through fsq_append, x ~ N(0,1) bf16 drawn per
        chunk from its own seed [workload, 0, T_X, chunk] (synth.layer_x_chunk,
        generated ahead by host threads); the layers get copies (timing does not
        depend on the code values). on_chunk(rows, x) sees every chunk's x (the
        CPU baseline's oracle encodes the same chunks into its own cache)."""
        from concurrent.futures import ThreadPoolExecutor
        E, _ = synth.layer_weights(w, 0)
        Ed = bf(E)
        codes = torch.empty((w.batch, w.context, w.P), dtype=torch.uint8, device="cuda")
        n = w.context // chunk
        assert w.batch == 1 and n * chunk == w.context
        ahead = 8
        with ThreadPoolExecutor(ahead) as ex:
            futs = [ex.submit(synth.layer_x_chunk, w, 0, c, chunk) for c in range(min(ahead, n))]
            for c in range(n):
                x = futs[c].result()
                futs[c] = None
                if c + ahead < n:
                    futs.append(ex.submit(synth.layer_x_chunk, w, 0, c + ahead, chunk))
                rows = slice(c * chunk, (c + 1) * chunk)
                self.fsq.fsq_append(bf(x), Ed, codes[0, rows])
                if on_chunk is not None:
                    on_chunk(rows, x)
        torch.cuda.synchronize()
        return codes

    def step_recon(self, r, rope=None):
        """One decode step through the key-reconstruction variant (no append);
        with rope = (gain, theta, eps), the Eq. 5 keys with norm and RoPE."""
        fsq, w = self.fsq, self.w
        for d in self.reps[r]:
            if rope is None:
                fsq.fsq_decode_attn_recon(d["q"], d["codes"], d["W"], self.lens, d["out"], w.n_kv,
                                          workspace=self.ws)
            else:
                fsq.fsq_decode_attn_rope(d["q"], d["codes"], d["W"], rope[0], self.lens, d["out"], w.n_kv,
                                         rope[1], rope[2], workspace=self.ws)

    def step(self, r, ev=None, two_call=False):
        """One decode step over replica r: per layer, one fsq_decode_step call
        (append of the new token at row T - 1 + attention; levels as the
        workload's codes). With ev (eager only),
        ev[l] = (start, stop) events bracket layer l's split-K kernel; that form
        issues the same work as fsq_append + fsq_decode_attn_timed (the split-K
        kernel and its inputs are the same)."""
        fsq, w = self.fsq, self.w
        for l, d in enumerate(self.reps[r]):
            if ev is None and not two_call:
                fsq.fsq_decode_step(d["x"], d["E"], d["q"], d["codes"], d["W"], self.lens, d["out"],
                                    w.n_kv, workspace=self.ws, levels=w.levels)
                continue
            if w.levels != 16:   # 2- / 8-bit codes, timed or two-call form: append + attention calls
                for b in range(w.batch):
                    T = int(self.lens_np[b])
                    fsq.fsq_append(d["x"][b:b + 1], d["E"], d["codes"][b, T - 1:T], levels=w.levels)
                fsq.fsq_decode_attn_levels(d["q"], d["codes"], d["W"], self.lens, d["out"], w.n_kv, w.levels,
                                           workspace=self.ws, split_events=None if ev is None else ev[l])
                continue
            for b in range(w.batch):
                T = int(self.lens_np[b])
                fsq.fsq_append(d["x"][b:b + 1], d["E"], d["codes"][b, T - 1:T])
            fsq.fsq_decode_attn(d["q"], d["codes"], d["W"], self.lens, d["out"], w.n_kv,
                                workspace=self.ws, split_events=None if ev is None else ev[l])


def run_workload(w, torch, steps, warmup, eager, timing_steps, two_call=False, on_chunk=None):
    per_step_bytes = w.layers * (decode_call_bytes(w, synth.seq_lens(w)) + append_call_bytes(w))
    replicas = max(2, math.ceil(4 * MALL_BYTES / per_step_bytes))
    replicas = min(replicas, 8)
    m = Model(w, torch, replicas, on_chunk)
    graphs = None
    if not eager:
        stream = torch.cuda.Stream()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            for r in range(replicas):     # warm the library and the allocator outside capture
                m.step(r, two_call=two_call)
        torch.cuda.current_stream().wait_stream(stream)
        torch.cuda.synchronize()
        graphs = []
        for r in range(replicas):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                m.step(r, two_call=two_call)
            graphs.append(g)

    def run(i):
        r = i % replicas
        if graphs is not None:
            graphs[r].replay()
        else:
            m.step(r, two_call=two_call)

    # phase A: throughput of whole steps (graph replays, inputs resident in HBM)
    for i in range(warmup):
        run(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        run(warmup + i)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps

    # phase A2: the same steps again, one event pair per step, for the spread
    per = []
    for i in range(steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        run(warmup + steps + i)
        b.record()
        per.append((a, b))
    torch.cuda.synchronize()
    step_ms = [a.elapsed_time(b) for a, b in per]

    # phase B: eager steps with HIP events around every split-K kernel launch
    call_ms = []
    for i in range(timing_steps):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(w.layers)]
        m.step((warmup + steps + i) % replicas, ev)
        torch.cuda.synchronize()
        call_ms.extend(a.elapsed_time(b) for a, b in ev)
    return m, ms, call_ms, replicas, step_ms


def step_spread(step_ms, seed=0, resamples=2000):
    """Median of per-step times with a 95% bootstrap interval of the median."""
    x = np.asarray(step_ms, dtype=np.float64)
    g = np.random.default_rng(seed)
    med = np.median(g.choice(x, size=(resamples, x.size), replace=True), axis=1)
    return {"median_ms": float(np.median(x)), "ci95_ms": [float(np.percentile(med, 2.5)), float(np.percentile(med, 97.5))],
            "steps": int(x.size), "timing": "one event pair per graph-replayed step"}


def append_prefill(w, torch, calls=40, eager=False):
    """fsq_append of the workload's prefill chunk (x [n, C] -> codes [n, P]), replayed
    from a HIP graph (or launched eagerly) over replicas of x that together exceed
    the Infinity Cache; returns the average time per call and its HBM roofline."""
    import fsq_latent_decode_amd as fsq
    n = w.append_tokens
    E, _ = synth.layer_weights(w, 0)
    x_bits = synth.layer_x(w, 0, n)
    to_dev = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).cuda()
    x0 = to_dev(x_bits)
    reps = max(2, math.ceil(4 * MALL_BYTES / x0.numel() / 2))
    xs = [x0] + [x0.clone() for _ in range(reps - 1)]
    Ed = to_dev(E)
    codes = [torch.empty((n, w.P), dtype=torch.uint8, device="cuda") for _ in range(reps)]
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for r in range(reps):
            fsq.fsq_append(xs[r], Ed, codes[r])
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    def all_calls():
        for i in range(calls):
            fsq.fsq_append(xs[i % reps], Ed, codes[i % reps])
    if eager:
        run = all_calls
    else:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            all_calls()
        run = g.replay
    run()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    run()
    t1.record()
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1e3 / calls
    nbytes = n * w.C * 2 + w.G * w.C * 2 + n * w.P
    flops = 2.0 * n * w.G * w.C
    ach = nbytes / (us * 1e-6) / 1e9
    codes0 = codes[0].cpu().numpy()
    floor = append_load_floor(w, torch, xs, Ed, calls)
    return codes0, {"workload": w.name, "tokens": n, "C": w.C, "G": w.G, "us_per_call": us,
            "tokens_per_s": n / (us * 1e-6),
            "roofline": {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": ach / HBM_PEAK_GBS, "bytes_per_call": nbytes,
                         "mfma_frac": flops / (us * 1e-6) / (MFMA_FP16_PEAK_TFLOPS * 1e12)},
            "traffic": traffic_from_append_profile(w),
            "load_floor": floor,
            "timing": (f"{calls} eager calls" if eager else f"{calls} calls in one HIP graph")
                      + f" over {reps} replicas of x, events around them"}


def append_load_floor(w, torch, xs, Ed, calls):
    """The prefill append's memory side alone: a load-only kernel (the probe
    library built beside libfsq.so) that issues the append kernel's per-CU reads
    of x and of E, timed like the append (HIP graph of `calls` launches over the
    replicas of x): x and E together, x alone, E alone."""
    import ctypes
    path = os.path.join(ROOT, "fsq_latent_decode_amd", "lib", "libfsq_probe.so")
    if not os.path.exists(path):
        return {"skipped": "libfsq_probe.so not built"}
    lib = ctypes.CDLL(path)
    lib.fsq_probe_append_loads.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                           ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.fsq_probe_append_loads.restype = ctypes.c_int
    n = xs[0].shape[0]
    out = torch.empty((n // 32) * 512, dtype=torch.int32, device="cuda")
    res = {"what": "load-only kernel with the append's per-CU reads (32 tokens per CTA: the CTA's x rows "
                   "and all GP rows of E, 512-byte row segments, rotated batch order, 16 loads in flight "
                   "per wave)"}
    for mode, key in ((0, "x_and_E_us"), (1, "x_only_us"), (2, "E_only_us")):
        def launch(i):
            rc = lib.fsq_probe_append_loads(mode, xs[i % len(xs)].data_ptr(), Ed.data_ptr(), n, w.C, w.G,
                                            out.data_ptr(), torch.cuda.current_stream().cuda_stream)
            if rc != 0:
                raise RuntimeError(f"fsq_probe_append_loads returned {rc}")
        for i in range(len(xs)):
            launch(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(calls):
                launch(i)
        g.replay()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        g.replay()
        t1.record()
        torch.cuda.synchronize()
        res[key] = t0.elapsed_time(t1) * 1e3 / calls
    return res


def launch_floor(w, torch, kernels_per_layer=3, steps=30):
    """Time a step's launch chain alone: layers x kernels_per_layer dependent
    trivial kernels (fill_ of a 512 KB buffer, 256 CTAs each) replayed from one
    HIP graph, the step's own launch pattern with no work behind it."""
    bufs = [torch.empty(256 * 512, dtype=torch.float32, device="cuda") for _ in range(kernels_per_layer)]
    def chain():
        for l in range(w.layers):
            for i, b in enumerate(bufs):
                b.fill_(float(l * kernels_per_layer + i))
    chain()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        chain()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    n = w.layers * kernels_per_layer
    return {"what": f"{w.layers} layers x {kernels_per_layer} dependent trivial kernels (256 CTAs each) "
                    "in one HIP graph: the step's launch chain without its work",
            "kernels_per_step": n, "ms_per_step": ms, "us_per_kernel": ms * 1e3 / n}


def copy_probe(torch, mib):
    n = mib * 2 ** 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "dispatches": 3}))


# --------------------------------------------------------------- CPU side
class OracleCache:
    """The oracle's own cache of a workload whose codes are FSQ(E x) (the
    million-token workload): Model.fsq_cache hands it every prefill chunk's x,
    the oracle encodes it (Eq. 2 and 4 in fp64) into its rows. Only the CPU
    baseline leg uses it."""

    def __init__(self, w):
        from oracle import fsq_oracle as orc
        self.orc, self.w = orc, w
        E, _ = synth.layer_weights(w, 0)
        self.Ef = synth.bf16_bits_to_f64(E)
        self.codes = np.empty((1, w.context, w.P), np.uint8)
        self.seconds = 0.0

    def __call__(self, rows, x):
        t = time.perf_counter()
        self.codes[0, rows] = self.orc.pack_codes(self.orc.encode(synth.bf16_bits_to_f64(x), self.Ef))
        self.seconds += time.perf_counter() - t


def cpu_baseline(w, seconds, gpu_out=None, ref_codes=None, max_layers=None):
    """The fp64 oracle (oracle/) as it stands, on a bounded sample of the step:
    whole layers (one-token append + decode at full context), extrapolated to
    the workload's layer count; timed with the BLAS threads available and with
    one thread. With gpu_out (layer -> the GPU's output of that layer in the
    timed steps) the oracle's outputs of the sampled layers are compared with
    it (relative L2 per layer and the worst per head). ref_codes: the oracle's
    own cache of layer 0 (codes from FSQ(E x), OracleCache); the sample is then
    that one layer."""
    from oracle import fsq_oracle as orc
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threadpool_limits = None
        threads = 1
    lens = synth.seq_lens(w)
    if ref_codes is not None:
        max_layers = 1

    def inputs(l):
        E, W = synth.layer_weights(w, l)
        codes = (ref_codes.copy() if ref_codes is not None
                 else synth.layer_codes(w, l, lens=lens if w.ragged else None))
        return (synth.bf16_bits_to_f64(synth.layer_x(w, l, w.batch, synth.T_XNEW)),
                synth.bf16_bits_to_f64(synth.layer_query(w, l)), codes,
                synth.bf16_bits_to_f64(W), synth.bf16_bits_to_f64(E))

    def layer(x, q, packed, Wf, Ef):
        new = orc.pack_codes(orc.encode(x, Ef))
        for b in range(w.batch):
            packed[b, int(lens[b]) - 1] = new[b]
        return orc.decode_attn(q, packed, Wf, lens, w.n_kv, w.G)

    def run(budget, keep):
        # layers in order, wrapping to further steps until the time budget is
        # spent (the inputs of a layer are the same in every step)
        done, t_total, outs = 0, 0.0, {}
        while t_total < budget and (max_layers is None or done < max_layers):
            args = inputs(done % w.layers)
            t = time.perf_counter()
            out = layer(*args)
            t_total += time.perf_counter() - t
            if keep and done < w.layers:
                outs[done] = out
            done += 1
        return done, t_total, outs

    done, t_total, outs = run(seconds, True)
    per_step = t_total / done * w.layers
    res = {"value": float(np.sum(lens)) / per_step, "unit": "context-tokens/s", "cores": threads,
           "kind": "oracle",
           "sample": f"{done} layer(s) ({done / w.layers:.2f} steps of {w.layers} layers; one-token append + "
                     f"decode at full context), {t_total:.1f} s of oracle time, scaled to one step",
           "step_s": per_step, "cpu_count": os.cpu_count(),
           "affinity_cores": len(os.sched_getaffinity(0))}
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            d1, t1, _ = run(seconds / 2, False)
        res["one_thread"] = {"value": float(np.sum(lens)) / (t1 / d1 * w.layers), "layers": d1,
                             "seconds": t1}
    if gpu_out:
        errs, heads = [], []
        for l in sorted(outs):
            if l not in gpu_out:
                continue
            g, o = gpu_out[l], outs[l]
            live = np.asarray(lens) > 0
            errs.append(float(np.linalg.norm(g - o) / np.linalg.norm(o)))
            hr = np.linalg.norm(g - o, axis=-1) / np.maximum(np.linalg.norm(o, axis=-1), 1e-30)
            heads.append(float(hr[live].max()))
        res["parity"] = {"layers": len(errs), "max_rel_l2": max(errs) if errs else None,
                         "max_head_rel_l2": max(heads) if heads else None, "bar": 5e-3,
                         "what": "GPU output of the timed steps vs the oracle, same layers"
                                 + ("; the oracle decodes its own cache of the same FSQ(E x) chunks"
                                    if ref_codes is not None else "")}
    return res


def cpu_append_baseline(w, gpu_codes, seconds=3.0):
    """The oracle's encode (Eq. 4 with the Eq. 2 forward value, fp64, then
    packing) of the workload's prefill chunk, repeated for about `seconds`; its
    codes are compared with the GPU's append of the same chunk (codes may differ
    by +-1 only at fp32 rounding ties: the count and largest difference are
    reported)."""
    from oracle import fsq_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    n = w.append_tokens
    E, _ = synth.layer_weights(w, 0)
    xf = synth.bf16_bits_to_f64(synth.layer_x(w, 0, n))
    Ef = synth.bf16_bits_to_f64(E)
    reps, t_total, ref = 0, 0.0, None
    while t_total < seconds or reps == 0:
        t = time.perf_counter()
        ref = orc.encode(xf, Ef)
        orc.pack_codes(ref)
        t_total += time.perf_counter() - t
        reps += 1
    got = orc.unpack_codes(gpu_codes, w.G)
    diff = np.abs(got.astype(int) - ref.astype(int))
    return {"value": n * reps / t_total, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} encodes of the {n}-token chunk, {t_total:.1f} s",
            "parity": {"codes": int(ref.size), "differing": int(np.count_nonzero(diff)),
                       "max_abs_diff": int(diff.max()), "bar": "at most 1e-4 of codes, each by +-1"}}


def split_kernel_bytes(w, lens):
    """Algorithmic bytes of one split-K launch: the layer's packed codes."""
    return int(np.sum(lens)) * w.P


DECODE_SRC = ("decode.hip", "common.h", "decode_plan.h")
APPEND_SRC = ("append.hip", "common.h", "append_gemv.h")


def kernel_src_sha(files):
    """sha256 over the kernel sources (under the package's csrc/, in order) that a
    counter summary was taken on."""
    import hashlib
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, "fsq_latent_decode_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def _profile_bytes(path, files):
    """hbm_bytes_per_dispatch of a committed rocprofv3 counter summary, if it was
    taken on the current sources; else None (the counters no longer describe the
    kernel)."""
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_src_sha256") != kernel_src_sha(files):
        return None
    try:
        return float(kv["hbm_bytes_per_dispatch"])
    except (KeyError, ValueError):
        return None


def graph_replayed_split_us(w):
    """The split-K kernel's average duration over graph-replayed launches, from
    the committed rocprofv3 kernel trace of the same sources (HIP events cannot
    be recorded inside a captured graph, so the live measurement is eager)."""
    for f in sorted(os.listdir(os.path.join(ROOT, "profiles"))):
        if not f.startswith("decode_step_kernels_"):
            continue
        kv = {}
        for line in open(os.path.join(ROOT, "profiles", f)):
            if "=" in line and not line.startswith(("#", "|")):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
        if kv.get("kernel_src_sha256") == kernel_src_sha(DECODE_SRC) and f"split_k_graph_avg_us.{w.name}" in kv:
            return float(kv[f"split_k_graph_avg_us.{w.name}"]), f
    return None, None


def traffic_from_profile(w):
    """HBM bytes per split-K launch from the committed counter summary."""
    return _profile_bytes(os.path.join(ROOT, "profiles", f"decode_split_traffic_{w.name}.txt"), DECODE_SRC)


def traffic_from_append_profile(w):
    """HBM bytes per prefill-append launch from the committed counter summary."""
    return _profile_bytes(os.path.join(ROOT, "profiles", f"append_prefill_traffic_{w.name}.txt"), APPEND_SRC)


def sdpa_comparison(w, torch, fsq_ms, steps=10, warmup=3):
    """The same decode step over materialised bf16 K = Z W_k^T and V = Z W_v^T
    (4 * n_kv * d_h bytes per token and layer) through PyTorch's fused SDPA,
    timed like the FSQ steps (HIP graph of all layers, inputs resident). The
    query heads of a kv head ride as rows of one attention (GQA without copies).
    Only PyTorch's flash / memory-efficient backends are allowed; if neither
    takes these shapes the comparison reports why instead of running the
    unfused path. The layer-0 output is compared with fsq_decode_attn's on the
    same codes."""
    import torch.nn.functional as F
    from torch.nn.attention import SDPBackend, sdpa_kernel
    import fsq_latent_decode_amd as fsq
    if w.ragged or w.codes_from_fsq:
        return None
    lens = synth.seq_lens(w)
    T = int(lens[0])
    grp = w.n_q // w.n_kv
    to_bf = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).cuda()
    layers = []
    for l in range(w.layers):
        _, Wb = synth.layer_weights(w, l)
        codes = torch.from_numpy(synth.layer_codes(w, l)).cuda()          # [B, T, P]
        z = torch.stack([codes & 15, codes >> 4], dim=-1).reshape(w.batch, T, -1)[..., :w.G]
        z = z.float() - 8.0                                                # [B, T, G]
        Wf = to_bf(Wb).float()
        Wk = Wf[: w.n_kv * w.d_h].reshape(w.n_kv, w.d_h, w.G)
        Wv = Wf[w.n_kv * w.d_h:].reshape(w.n_kv, w.d_h, w.G)
        zz = z.unsqueeze(1)                                                # [B, 1, T, G] fp32
        K = torch.matmul(zz, Wk.transpose(1, 2).contiguous().unsqueeze(0)).to(torch.bfloat16).contiguous()
        V = torch.matmul(zz, Wv.transpose(1, 2).contiguous().unsqueeze(0)).to(torch.bfloat16).contiguous()
        qb = to_bf(synth.layer_query(w, l))                                # [B, n_q, d_h]
        q = qb.reshape(w.batch, w.n_kv, grp, w.d_h).contiguous()
        layers.append(dict(q=q, q1=qb.reshape(w.batch, w.n_q, 1, w.d_h).contiguous(), K=K, V=V, qb=qb,
                           W=to_bf(Wb), codes=codes))
        del z, zz, Wf
    backends = [SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION]
    kv_bytes = w.layers * w.batch * T * 4 * w.n_kv * w.d_h
    res = {"workload": w.name, "kv_bytes_per_token_per_layer": 4 * w.n_kv * w.d_h,
           "fsq_bytes_per_token_per_layer": w.P, "kv_bytes_per_step": kv_bytes,
           "materialised_hbm_roofline_ms": kv_bytes / (HBM_PEAK_GBS * 1e9) * 1e3,
           "fsq_ms_per_step": fsq_ms, "backends_allowed": "flash, memory-efficient", "forms": {}}
    best = None
    for form in ("grouped_rows", "enable_gqa", "matmul_softmax"):
        r = _time_sdpa(torch, F, sdpa_kernel, backends, layers, form, steps, warmup)
        res["forms"][form] = r
        if "ms_per_step" in r and (best is None or r["ms_per_step"] < res["forms"][best]["ms_per_step"]):
            best = form
    if best is None:
        return res
    ms = res["forms"][best]["ms_per_step"]
    ach = kv_bytes / (ms * 1e-3) / 1e9
    d0 = layers[0]
    mine = torch.empty((w.batch, w.n_q, w.d_h), dtype=torch.bfloat16, device="cuda")
    fsq.fsq_decode_attn(d0["qb"], d0["codes"], d0["W"], torch.from_numpy(lens).cuda(), mine, w.n_kv)
    torch.cuda.synchronize()
    a = res["forms"][best].pop("_out0").reshape(w.batch, w.n_q, w.d_h).double()
    for r in res["forms"].values():
        r.pop("_out0", None)
    b = mine.double()
    res.update({"best_form": best, "ms_per_step": ms,
                "context_tokens_per_s": float(np.sum(lens)) / (ms * 1e-3),
                "achieved_GBs": ach, "hbm_frac": ach / HBM_PEAK_GBS, "fsq_speedup": ms / fsq_ms,
                "layer0_rel_l2_sdpa_vs_fsq": float(torch.linalg.norm(a - b) / torch.linalg.norm(b))})
    del layers
    torch.cuda.empty_cache()
    return res


def _time_sdpa(torch, F, sdpa_kernel, backends, layers, form, steps, warmup):
    """Time one step of attention calls over all layers; form "grouped_rows"
    puts the query heads of a kv head as rows of one SDPA call, "enable_gqa"
    passes all query heads with PyTorch's GQA flag, "matmul_softmax" is
    unfused: bf16 library products S = K q^T and out = P^T V (contiguous
    operands) around an fp32 softmax over the whole context."""
    res = {}
    outs = []
    for d in layers:
        outs.append(torch.empty_like(d["q"] if form != "enable_gqa" else d["q1"]))
        if form == "matmul_softmax":
            d["qT"] = d["q"].transpose(-1, -2).contiguous()                 # [B, n_kv, d_h, grp]
    scale = 1.0 / math.sqrt(layers[0]["q"].shape[-1])

    def step():
        for d, o in zip(layers, outs):
            if form == "grouped_rows":
                o.copy_(F.scaled_dot_product_attention(d["q"], d["K"], d["V"]))
            elif form == "enable_gqa":
                o.copy_(F.scaled_dot_product_attention(d["q1"], d["K"], d["V"], enable_gqa=True))
            else:
                sc = torch.matmul(d["K"], d["qT"]).float() * scale          # [B, n_kv, T, grp]
                p = torch.softmax(sc, dim=2).to(torch.bfloat16)
                o.copy_(torch.matmul(p.transpose(-1, -2).contiguous(), d["V"]))

    try:
        with sdpa_kernel(backends):
            step()
            torch.cuda.synchronize()
            graph = None
            try:
                s = torch.cuda.Stream()
                s.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(s):
                    step()
                torch.cuda.current_stream().wait_stream(s)
                torch.cuda.synchronize()
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(graph):
                    step()
            except Exception as e:  # noqa: BLE001 - fall back to eager launches
                graph = None
                res["graph_error"] = str(e)[:200]
            run = graph.replay if graph is not None else step
            for _ in range(warmup):
                run()
            torch.cuda.synchronize()
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0.record()
            for _ in range(steps):
                run()
            t1.record()
            torch.cuda.synchronize()
    except RuntimeError as e:
        res["unavailable"] = str(e)[:300]
        return res
    res.update({"ms_per_step": t0.elapsed_time(t1) / steps,
                "timing": ("HIP graph of all layers" if "graph_error" not in res else "eager launches")
                          + f", {steps} steps", "_out0": outs[0]})
    return res


def layer_batched(w, torch, steps=10, warmup=3):
    """Not the model's call pattern: the attention of all the workload's layers in
    ONE fsq_decode_attn call, the layers' caches and queries taken as a batch of
    sequences under layer 0's W_kv. It shows the decode kernels with the GPU
    filled (the per-layer calls of a decode step are bound by launch and
    dependent-load latency); the same bytes and flops per layer as the step.
    Replicas exceed the Infinity Cache; graph-replayed; then eager calls with
    events around the split-K kernel."""
    import fsq_latent_decode_amd as fsq
    if w.batch != 1 or w.levels != 16:
        return None
    L, T = w.layers, int(w.context)
    lens_np = np.full(L, T, dtype=np.int32)
    nbytes = L * T * w.P
    replicas = min(4, max(2, math.ceil(4 * MALL_BYTES / nbytes)))
    dev = "cuda"
    _, W = synth.layer_weights(w, 0)
    Wd = torch.from_numpy(np.ascontiguousarray(W).view(np.int16)).view(torch.bfloat16).to(dev)
    qs = np.concatenate([synth.layer_query(w, l) for l in range(L)], axis=0)
    q = torch.from_numpy(np.ascontiguousarray(qs).view(np.int16)).view(torch.bfloat16).to(dev)
    lens = torch.from_numpy(lens_np).to(dev)
    reps = []
    for r in range(replicas):
        g = torch.Generator(device=dev)
        g.manual_seed(7_000_001 * w.wid + r)
        codes = torch.randint(0, 256, (L, T, w.P), generator=g, device=dev, dtype=torch.int32).to(torch.uint8)
        reps.append((codes, torch.empty((L, w.n_q, w.d_h), dtype=torch.bfloat16, device=dev)))
    ws = fsq.alloc_workspace(L, w.n_q, w.G, T, dev)
    plan = fsq.decode_plan(L, w.n_q, w.G, T)
    call = lambda r, ev=None: fsq.fsq_decode_attn(q, reps[r][0], Wd, lens, reps[r][1], w.n_kv, workspace=ws,
                                                  split_events=ev)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for r in range(replicas):
            call(r)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graphs = []
    for r in range(replicas):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            call(r)
        graphs.append(gr)
    for i in range(warmup):
        graphs[i % replicas].replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        graphs[(warmup + i) % replicas].replay()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    ks = []
    for i in range(5):
        ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        call(i % replicas, ev)
        torch.cuda.synchronize()
        ks.append(ev[0].elapsed_time(ev[1]))
    k_ms = float(np.mean(ks))
    del reps, graphs, ws
    torch.cuda.empty_cache()
    return {"what": f"all {L} layers' attention in one call: {L} caches and queries as a batch under one W_kv "
                    "(not the model's call pattern, which is one dependent call per layer)",
            "ms_per_call": ms, "context_tokens_per_s": L * T / (ms * 1e-3),
            "kernel": plan["kernel"], "device_split": plan["device_split"],
            "split_kernel_us": k_ms * 1e3,
            "roofline": {"bound": "hbm", "achieved": nbytes / (k_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": nbytes / (k_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                         "bytes_per_launch": nbytes},
            "call_roofline_frac": (nbytes / (HBM_PEAK_GBS * 1e9)) / (ms * 1e-3)}


def recon_comparison(w, torch, fsq_ms, steps=10, warmup=3, rope=False):
    """The decode step with keys rebuilt per tile (fsq_decode_attn_recon; with
    rope, fsq_decode_attn_rope: key RMS norm with a seeded gain, eps 1e-6, and
    RoPE with theta 1e6) on the same replicated inputs, graph-replayed like the
    FSQ steps. The path is bound by its MFMA work: 2 n_kv d_h G flops per token
    for the keys, against the absorbed path's 2 n_q G for the scores (pooling
    and W_v are common)."""
    if w.d_h % 32 or w.d_h > 128 or (rope and w.d_h not in (64, 128)):
        return None
    lens = synth.seq_lens(w)
    per_step_bytes = w.layers * decode_call_bytes(w, lens)
    replicas = min(8, max(2, math.ceil(4 * MALL_BYTES / per_step_bytes)))
    m = Model(w, torch, replicas)
    rp = None
    if rope:
        gam = synth.normal_bf16(synth.rng(w.wid, 0, 301), (w.d_h,), 0.1)
        gam = synth.f32_to_bf16_bits(synth.bf16_bits_to_f64(gam).astype(np.float32) + 1.0)
        rp = (torch.from_numpy(gam.view(np.int16)).view(torch.bfloat16).cuda(), 1e6, 1e-6)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for r in range(replicas):
            m.step_recon(r, rp)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graphs = []
    for r in range(replicas):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            m.step_recon(r, rp)
        graphs.append(g)
    for i in range(warmup):
        graphs[i % replicas].replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        graphs[(warmup + i) % replicas].replay()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    ctx = float(np.sum(lens))
    key_flops = 2.0 * w.layers * ctx * w.n_kv * w.d_h * w.G
    common = 2.0 * w.layers * ctx * w.n_q * (w.d_h + w.G)     # scores on rebuilt keys + pooling
    flops = key_flops + common
    absorbed = 2.0 * w.layers * ctx * w.n_q * w.G * 2
    tf = flops / (ms * 1e-3) / 1e12
    del m, graphs
    torch.cuda.empty_cache()
    return {"workload": w.name, "keys": ("RoPE_t(N_k(W_k z)), theta 1e6, eps 1e-6" if rope else "W_k z"),
            "ms_per_step": ms, "context_tokens_per_s": ctx / (ms * 1e-3),
            "fsq_ms_per_step": fsq_ms, "slowdown_vs_absorbed": ms / fsq_ms,
            "flops_per_step": flops, "absorbed_path_flops_per_step": absorbed,
            "roofline": {"bound": "mfma", "achieved": tf, "peak": MFMA_FP16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": tf / MFMA_FP16_PEAK_TFLOPS,
                         "t_roof_ms": flops / (MFMA_FP16_PEAK_TFLOPS * 1e12) * 1e3},
            "timing": f"{steps} steps from HIP graphs over {replicas} replicas (no append)"}


def summarize(w, ms, call_ms, replicas):
    lens = synth.seq_lens(w)
    ctx = float(np.sum(lens))
    step_bytes = w.layers * (decode_call_bytes(w, lens) + append_call_bytes(w))
    t_bytes = step_bytes / (HBM_PEAK_GBS * 1e9)
    t_flops = step_flops(w, lens) / (MFMA_FP16_PEAK_TFLOPS * 1e12)
    t_roof = max(t_bytes, t_flops)
    res = {"value": ctx / (ms * 1e-3), "ms_per_step": ms, "steps_per_s": 1e3 / ms,
           "step_roofline": {"bytes": step_bytes, "flops": step_flops(w, lens),
                             "t_roof_us": t_roof * 1e6, "frac": t_roof / (ms * 1e-3)},
           "replicas": replicas}
    if call_ms:
        import fsq_latent_decode_amd as fsq
        plan = fsq.decode_plan(w.batch, w.n_q, w.G, int(w.context))
        avg = float(np.mean(call_ms))
        nbytes = split_kernel_bytes(w, lens)
        ach = nbytes / (avg * 1e-3) / 1e9
        split = ({"split": "on the device from the lengths", "splits_per_sequence_max": plan["splits"],
                  "chunk_tokens_min": plan["chunk"]} if plan["device_split"] else
                 {"split": "host plan", "splits_per_sequence": plan["splits"], "chunk_tokens": plan["chunk"]})
        res["roofline"] = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": ach / HBM_PEAK_GBS, "traffic": traffic_from_profile(w),
                           "kernel": plan["kernel"], **split, "bytes_per_launch": nbytes,
                           "avg_launch_us": avg * 1e3, "launches_timed": len(call_ms),
                           "timing": "hipExtLaunchKernelGGL start/stop events, eager steps"}
        g_us, g_src = graph_replayed_split_us(w)
        if g_us is not None:
            g_ach = nbytes / (g_us * 1e-6) / 1e9
            res["roofline"]["graph_replayed"] = {"avg_launch_us": g_us, "achieved": g_ach,
                                                 "frac": g_ach / HBM_PEAK_GBS,
                                                 "timing": f"rocprofv3 kernel trace of the graph-replayed steps "
                                                           f"(profiles/{g_src}), same sources"}
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path would shard by sequence; see the design notes)", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_probe_mib:
        copy_probe(torch, args.copy_probe_mib)
        return
    if args.append_only:
        name = next(n for n in [args.workload] + [s for s in args.also.split(",") if s]
                    if synth.WORKLOADS[n].append_tokens)
        print(json.dumps(append_prefill(synth.WORKLOADS[name], torch, calls=12 if args.eager else 40,
                                        eager=args.eager)[1]))
        return
    w = synth.WORKLOADS[args.workload]
    cpu_on = not args.no_cpu_baseline
    oracle_caches = {}

    def on_chunk_for(wk):
        if not (cpu_on and wk.codes_from_fsq and wk.name in CPU_BASELINE_WORKLOADS):
            return None
        oracle_caches[wk.name] = OracleCache(wk)
        return oracle_caches[wk.name]

    def outputs(m, wk):
        # the GPU's outputs of the timed steps (replica 0), every layer
        return {l: d["out"].float().cpu().numpy().astype(np.float64) for l, d in enumerate(m.reps[0])}

    m, ms, call_ms, reps, step_ms = run_workload(w, torch, args.steps, args.warmup, args.eager,
                                                 args.timing_steps, args.two_call, on_chunk_for(w))
    main_res = summarize(w, ms, call_ms, reps)
    main_res["step_spread"] = step_spread(step_ms)
    gpu_out = outputs(m, w)
    del m
    torch.cuda.empty_cache()
    also, also_out = {}, {}
    for name in [s for s in args.also.split(",") if s and s != args.workload]:
        w2 = synth.WORKLOADS[name]
        m2, ms2, cm2, reps2, sm2 = run_workload(w2, torch, max(5, args.steps // 2), args.warmup,
                                                args.eager, args.timing_steps, args.two_call, on_chunk_for(w2))
        also[name] = summarize(w2, ms2, cm2, reps2)
        also[name]["step_spread"] = step_spread(sm2)
        if name in CPU_BASELINE_WORKLOADS:
            also_out[name] = outputs(m2, w2)
        del m2
        torch.cuda.empty_cache()
    sdpa = {}
    if not args.no_sdpa:
        fsq_ms = {w.name: main_res["ms_per_step"], **{k: v["ms_per_step"] for k, v in also.items()}}
        for name in [n for n in [args.workload] + [s for s in args.also.split(",") if s] if n in COMPARED]:
            r = sdpa_comparison(synth.WORKLOADS[name], torch, fsq_ms[name])
            if r is not None:
                sdpa[name] = r
    recon = {}
    if not args.no_recon:
        fsq_ms = {w.name: main_res["ms_per_step"], **{k: v["ms_per_step"] for k, v in also.items()}}
        for name in [n for n in [args.workload] + [s for s in args.also.split(",") if s] if n in COMPARED]:
            w2 = synth.WORKLOADS[name]
            r = recon_comparison(w2, torch, fsq_ms[name])
            if r is not None:
                recon[name] = r
            r = recon_comparison(w2, torch, fsq_ms[name], rope=True)
            if r is not None:
                recon[name + "_rope"] = r
    floor = None if args.no_launch_floor else launch_floor(w, torch)
    batched = {}
    if not args.no_layer_batched:
        for name in [n for n in [args.workload] + [s for s in args.also.split(",") if s] if n in COMPARED]:
            r = layer_batched(synth.WORKLOADS[name], torch)
            if r is not None:
                batched[name] = r
    app = None
    for name in [args.workload] + [s for s in args.also.split(",") if s]:
        if synth.WORKLOADS[name].append_tokens and not args.no_append:
            app_codes, app = append_prefill(synth.WORKLOADS[name], torch)
            if cpu_on:
                app["cpu_baseline"] = cpu_append_baseline(synth.WORKLOADS[name], app_codes)
            break
    cpu = None
    if cpu_on:
        oc = oracle_caches.get(w.name)
        cpu = cpu_baseline(w, args.cpu_seconds, gpu_out, ref_codes=None if oc is None else oc.codes)
        if oc is not None:
            cpu["reference_cache_encode_s"] = oc.seconds
        for name, outs2 in also_out.items():
            oc = oracle_caches.get(name)
            also[name]["cpu_baseline"] = cpu_baseline(synth.WORKLOADS[name], args.cpu_seconds * 2 / 3, outs2,
                                                      ref_codes=None if oc is None else oc.codes)
            if oc is not None:
                also[name]["cpu_baseline"]["reference_cache_encode_s"] = oc.seconds
    line = {
        "metric": "decode context-tokens/s",
        "value": main_res["value"],
        "unit": "context-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": w.name, "layers": w.layers, "batch": w.batch,
                   "context": int(np.max(synth.seq_lens(w))), "G": w.G, "C": w.C, "n_q": w.n_q,
                   "n_kv": w.n_kv, "d_h": w.d_h, "bytes_per_token_per_layer": w.P,
                   "step": ("per layer: fsq_append of the new token + fsq_decode_attn" if args.two_call
                            else "per layer: fsq_decode_step (append of the new token + attention)")},
        "decode_steps_per_s": main_res["steps_per_s"],
        "step_roofline": main_res["step_roofline"],
        "step_spread": main_res["step_spread"],
        "roofline": main_res.get("roofline"),
        "cpu_baseline": cpu,
        "also": also,
        "append_prefill": app,
        "sdpa_comparison": sdpa,
        "recon_comparison": recon,
        "layer_batched": batched,
        "launch_floor": floor,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
