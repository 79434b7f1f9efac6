#!/usr/bin/env python3
"""Decode-step benchmark of the weight-absorbed MLA path on one MI355X.

A step is one pass of the whole hot path over one batch: the fused
mla_decode_step, which stores the new row of every sequence (position
cache_lens - 1) and then attends over rows 0 .. cache_lens - 1 (dense, ragged
or top-k); with --unfused, mla_cache_write followed by mla_decode.  Inputs are
seeded synthetic tensors with the workload's shapes; they are resident in
HBM before timing starts.  R replicas of every input rotate from step to step
so that the working set exceeds the 256 MB Infinity Cache (consecutive layers
of a real model do not share weights or caches either).

The headline workload is the largest single-GPU one, the ragged batch of 32
sequences of 1024..16384 rows (about 390 MB per step).  The other H = 128
workloads (B = 1 at T = 4096, the FP8 cache at T = 32768, top-2048 of 65536)
are timed in the same run with fewer steps and reported under "configs".

Timing: G consecutive steps (rotating over the replicas) are captured in one
HIP graph, as a model captures its layers together; the timed region replays
exactly K steps (K / G graph launches), bracketed by torch.cuda.synchronize().  Per-kernel durations
come from a second pass of K eager steps in which the library launches every
kernel with start/end HIP events stamped by the dispatch itself (the
mla_params trace_events hook), i.e. the same kernel start and end times a
kernel trace reports.  The dominant kernel's average duration gives the
roofline entry.  The CPU baseline times the oracle on a bounded sample of the
headline workload.

Prints one JSON line.
"""
import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
MALL_BYTES = 256 << 20
METRIC = "MLA decode tokens/s + latent-cache HBM GB/s (% of peak), H=128, T=4K–64K"
HEADLINE = "ragged_b32_h128_t16384"
EXTRA = ["dense_b1_h128_t4096", "fp8_b16_h128_t32768", "topk2048_b8_h128_t65536",
         # one GPU's 16 of 128 heads with two query tokens per sequence (shared tile work)
         "ragged_b32_h128_t16384:16:2"]
KERNELS = ["absorb", "attention", "combine", "uproj"]
FUSED = True  # --unfused: the row store runs as its own mla_cache_write kernel


class HipEvents:
    """hipEvent_t handles through the HIP runtime torch already loaded."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        evs = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            evs.append(e.value)
        return evs

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(e)


def sources_sha():
    """sha256 (16 hex digits) of the kernel sources, in the order `cat *.hip *.hpp` reads them."""
    import glob
    import hashlib
    d = os.path.join(ROOT, "mla_latent_kv_08_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(d, "*.hip"))) + sorted(glob.glob(os.path.join(d, "*.hpp"))):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def counter_traffic(workload, kernel_symbol, check_sources=True):
    """HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE summary
    (first row of the workload whose symbol starts with `kernel_symbol`), or None
    when there is none for this kernel or the sources changed since."""
    import re
    path = os.path.join(ROOT, "profiles", "hbm_traffic_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"Sources at sha256 \(csrc/\*\.hip, \*\.hpp\) `([0-9a-f]+)`", text)
    if check_sources and (not m or m.group(1) != sources_sha()):
        return None
    for line in text.splitlines():
        cells = [c.strip().strip("`") for c in line.strip().strip("|").split("|")]
        if len(cells) == 6 and cells[0] == workload and cells[1].startswith(kernel_symbol):
            return int(float(cells[5]))
    return None


def stream_probe(torch, nbytes=2 << 30, reps=10, groups=2048):
    """Attainable HBM read bandwidth measured in this run: a read-only
    streaming kernel (16-byte non-temporal loads, each workgroup its own
    contiguous slice, nothing written back but one word per wavefront) over
    `nbytes`, far beyond the 256 MB Infinity Cache, timed with events over
    `reps` launches on the current stream; bytes read per second, in GB/s."""
    path = os.path.join(ROOT, "mla_latent_kv_08_amd", "libhbmprobe.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(path)
    lib.hbm_read_probe.restype = ctypes.c_int
    lib.hbm_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p,
                                   ctypes.c_void_p]
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda:0")
    sink = torch.zeros(4 * groups, dtype=torch.int32, device="cuda:0")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def launch():
        if lib.hbm_read_probe(buf.data_ptr(), nbytes, groups, sink.data_ptr(), stream) != 0:
            raise RuntimeError("hbm_read_probe launch failed")

    launch()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        launch()
    end.record()
    torch.cuda.synchronize()
    seconds = start.elapsed_time(end) * 1e-3 / reps
    del buf, sink
    return nbytes / seconds / 1e9


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def kernel_symbol(name, w):
    """The kernel's symbol as the profiles name it, or, for the attention kernel,
    the prefix up to its last template argument (heads per wave, which the work
    planner picks; a workload launches one instance)."""
    if name == "attention":
        return "mla::attn_kernel<%s, %s, " % ("true" if w.fp8 else "false", "true" if w.topk else "false")
    if name == "cache_write":
        return "mla::cache_write_fp8_kernel" if w.fp8 else "mla::cache_write_bf16_kernel"
    if name == "absorb":  # template argument: 0 no row store, 1 bf16 rows, 2 FP8 rows
        return "mla::absorb_kernel<%d>" % ((2 if w.fp8 else 1) if FUSED else 0)
    return {"combine": "mla::combine_kernel",
            "uproj": "mla::uproj_kernel"}[name]


def extra_workload(spec, synth, s_default):
    """An --extra entry: a workload name, or name:H:s for that workload with H
    heads and s query tokens per sequence (renamed <name>_h<H>).  Returns the
    workload and its s."""
    name, *over = spec.split(":")
    w, s = synth.WORKLOADS[name], s_default
    if over:
        heads = int(over[0])
        if len(over) > 1:
            s = int(over[1])
        if heads != w.heads:
            w = synth.scaled(w, heads=heads, name=f"{w.name}_h{heads}")
    return w, s


def workload_bytes_flops(w, lens, k, s=1):
    """Algorithmic bytes and FLOPs per kernel launch (one step).  With s query
    tokens per sequence the cache rows count once per sequence (the method
    scores all s tokens against them); the FLOPs count the rows each token sees
    (token i sees len - (s - 1 - i) rows)."""
    B, H = w.batch, w.heads
    Q = B * s  # query tokens
    rows = [min(k, int(n)) if k else int(n) for n in lens]
    tok_rows = [min(k, max(0, int(n) - (s - 1 - i))) if k else max(0, int(n) - (s - 1 - i))
                for n in lens for i in range(s)]
    row_bytes = (512 + 16 + 128) if w.fp8 else (1024 + 128)
    n_rows, n_tok_rows = sum(rows), sum(tok_rows)
    proj_w = 2 * H * 128 * 512
    out = {
        "absorb": (proj_w + 2 * Q * H * 128, 2 * Q * H * 128 * 512),
        "attention": (n_rows * row_bytes + 2 * Q * H * 64 + 4 * B + 4 * Q * k,
                      n_tok_rows * H * 2 * (576 + 512)),
        "combine": (0, 0),
        "uproj": (proj_w + 2 * Q * H * 128, 2 * Q * H * 128 * 512),
        "cache_write": (Q * 2 * 576 + Q * row_bytes + 4 * B, 0),
    }
    if FUSED:  # the row stores run inside the absorb launch
        out["absorb"] = (out["absorb"][0] + out.pop("cache_write")[0], out["absorb"][1])
    total_bytes = (2 * Q * H * 192 + 2 * proj_w + n_rows * row_bytes + 4 * B + 4 * Q * k
                   + 2 * Q * H * 128)
    total_flops = 4 * Q * H * 128 * 512 + n_tok_rows * H * 2 * (576 + 512)
    return out, total_bytes, total_flops, n_rows, row_bytes


def build_replicas(w, x, R, mla, torch):
    dev = "cuda:0"
    B, T = w.batch, w.max_seq_len
    s = x["q_nope"].shape[1]
    lens = x["cache_lens"]
    start = torch.clamp(lens - s, min=0)
    # the new rows are the cache's own last s rows, so every step stores the
    # same values again
    rows = (start.long().reshape(B, 1) + torch.arange(s).reshape(1, s)).clamp(max=T - 1)
    kv_new = x["kv"][torch.arange(B).reshape(B, 1), rows].reshape(B, s, 512).contiguous()
    pe_new = x["pe"][torch.arange(B).reshape(B, 1), rows].reshape(B, s, 64).contiguous()
    base = {
        "q_nope": x["q_nope"].to(dev), "q_pe": x["q_pe"].to(dev), "wkv_b": x["wkv_b"].to(dev),
        "kv_new": kv_new.to(dev), "pe_new": pe_new.to(dev),
    }
    if w.fp8:
        base["kv"] = torch.zeros(B, T, 512, dtype=torch.uint8, device=dev)
        base["scale"] = torch.zeros(B, T, 4, dtype=torch.float32, device=dev)
        base["pe"] = torch.zeros(B, T, 64, dtype=torch.bfloat16, device=dev)
        mla.cache_write(x["kv"].to(dev), x["pe"].to(dev), torch.zeros(B, dtype=torch.int32, device=dev),
                        base["kv"], base["pe"], kv_scale=base["scale"])
    else:
        base["kv"] = x["kv"].to(dev)
        base["scale"] = None
        base["pe"] = x["pe"].to(dev)
    shared = {"lens": lens.to(dev), "start": start.to(torch.int32).to(dev),
              "topk": None if x["topk_idx"] is None else x["topk_idx"].to(dev)}
    reps = [base]
    for _ in range(R - 1):
        reps.append({k: (None if v is None else v.clone()) for k, v in base.items()})
    torch.cuda.synchronize()
    return reps, shared


def step(mla, r, s, out, ws, trace=None):
    if FUSED:
        mla.decode_step(r["kv_new"], r["pe_new"], r["q_nope"], r["q_pe"], r["wkv_b"], r["kv"],
                        r["pe"], s["lens"], kv_scale=r["scale"], topk_idx=s["topk"], out=out,
                        workspace=ws, trace_events=None if trace is None else trace[1])
        return
    mla.cache_write(r["kv_new"], r["pe_new"], s["start"], r["kv"], r["pe"], kv_scale=r["scale"],
                    trace_events=None if trace is None else trace[0])
    mla.decode(r["q_nope"], r["q_pe"], r["wkv_b"], r["kv"], r["pe"], s["lens"], kv_scale=r["scale"],
               topk_idx=s["topk"], out=out, workspace=ws,
               trace_events=None if trace is None else trace[1])


def cpu_baseline(w, x, seconds, oracle, synth, np, torch):
    """The oracle, as it stands, on a bounded sample of the workload."""
    if w.fp8:
        kv, sc, pe = oracle.cache_write(x["kv"], x["pe"], torch.zeros(w.batch, dtype=torch.int32),
                                        w.max_seq_len, True)
    else:
        kv, sc, pe = x["kv"], None, x["pe"]
    Q = w.batch * x["q_nope"].shape[1]  # query tokens
    total_pairs = Q * w.heads
    pairs_all = [(q, h) for q in range(Q) for h in range(w.heads)]
    done, t0 = 0, time.perf_counter()
    chunk = max(1, min(total_pairs, 4 * oracle.num_threads()))
    i = 0
    while True:
        sel = [pairs_all[(i + j) % total_pairs] for j in range(chunk)]
        oracle.decode(x["q_nope"], x["q_pe"], x["wkv_b"], kv, pe, x["cache_lens"],
                      synth.SOFTMAX_SCALE, kv_scale=sc, topk_idx=x["topk_idx"], pairs=sel)
        done += chunk
        i += chunk
        el = time.perf_counter() - t0
        if el >= seconds and done >= min(total_pairs, chunk):
            break
    steps = done / total_pairs
    return {"value": Q * steps / el, "unit": "tokens/s", "cores": oracle.num_threads(),
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"{done} (query token, head) outputs of {w.name} in {el:.1f} s "
                      f"({steps:.3f} full steps; tokens/s = query tokens x steps / time)"}


def dtype_of(w):
    """Arithmetic type of the path: bf16 MFMA on bf16 rows; the FP8 cache is
    dequantised to bf16(code * scale) on the way into LDS and reaches the same
    bf16 MFMAs."""
    return "bf16" if not w.fp8 else "bf16 (fp8_e4m3 cache dequantised)"


def measure(w, args, steps, warmup, mla, synth, torch, np, S=1):
    """Times `steps` fused decode steps of workload `w` (graph replay) and the
    same number of eager steps with dispatch-stamped kernel events.  Returns
    (result fields, host inputs)."""
    x = synth.make_inputs(w)
    k = w.topk
    if S > 1:  # more query tokens per sequence: extra seeded draws of the same distributions
        x = synth.add_query_tokens(x, S, seed=w.seed + 1000)
    per_kernel, total_bytes, total_flops, n_rows, row_bytes = workload_bytes_flops(
        w, x["cache_lens"].tolist(), k, S)
    working = total_bytes + 2 * w.batch * w.heads * 128
    R = args.replicas or max(1, min(32, math.ceil(2 * MALL_BYTES / working)))
    reps, shared = build_replicas(w, x, R, mla, torch)
    B, H = w.batch, w.heads
    out = torch.empty(B, S, H, 128, dtype=torch.bfloat16, device="cuda:0")
    p = mla.make_params(B, H, w.max_seq_len, 1 if w.fp8 else 0, topk=k, seqlen_q=S)
    ws = torch.empty(mla.decode_workspace_size(p), dtype=torch.uint8, device="cuda:0")

    for i in range(warmup):
        step(mla, reps[i % R], shared, out, ws)
    torch.cuda.synchronize()

    # G consecutive steps per captured graph (as a model captures its layers
    # together), G dividing `steps`; step t uses replica t % R, so graph k of
    # L = lcm(G, R) / G distinct graphs covers the steps kG .. kG + G - 1
    G = args.graph_steps or max(d for d in range(1, 17) if steps % d == 0)
    if steps % G:
        raise SystemExit(f"--graph-steps {G} does not divide {steps} steps")
    L = R // math.gcd(G, R)
    graphs = []
    if not args.eager:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step(mla, reps[0], shared, out, ws)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        for k in range(L):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(G):
                    step(mla, reps[(k * G + i) % R], shared, out, ws)
            graphs.append(g)
        for i in range(max(1, warmup // G)):
            graphs[i % L].replay()
        torch.cuda.synchronize()

    # ---- timed region: exactly `steps` steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graphs:
        for k in range(steps // G):
            graphs[k % L].replay()
    else:
        for i in range(steps):
            step(mla, reps[i % R], shared, out, ws)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = 1e3 * elapsed / steps

    # ---- per-kernel durations: eager steps, start/end of every kernel stamped
    # by its dispatch
    hev = HipEvents()
    ev = hev.create(10 * steps)
    traces = []
    for i in range(steps):
        e = ev[10 * i: 10 * i + 10]
        traces.append(((ctypes.c_void_p * 2)(*e[:2]), (ctypes.c_void_p * 8)(*e[2:])))
    torch.cuda._sleep(int(2e8))  # let the host enqueue the steps ahead of the GPU
    for i in range(steps):
        step(mla, reps[i % R], shared, out, ws,
             trace=(ctypes.addressof(traces[i][0]), ctypes.addressof(traces[i][1])))
    torch.cuda.synchronize()
    dur = {kname: [] for kname in ([] if FUSED else ["cache_write"]) + KERNELS}
    for i in range(steps):
        e = ev[10 * i: 10 * i + 10]
        if not FUSED:
            dur["cache_write"].append(hev.elapsed_ms(e[0], e[1]))
        for j, kname in enumerate(KERNELS):
            dur[kname].append(hev.elapsed_ms(e[2 + 2 * j], e[3 + 2 * j]))
    hev.destroy(ev)
    del graphs, reps, shared, out, ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    avg_us = {kname: 1e3 * float(np.mean(v)) for kname, v in dur.items()}
    dom = max(avg_us, key=avg_us.get)
    kb, kf = per_kernel[dom]
    t_dom = avg_us[dom] * 1e-6
    hbm_time, mfma_time = kb / (PEAK_HBM_GBS * 1e9), kf / (PEAK_BF16_TFLOPS * 1e12)
    if hbm_time >= mfma_time:
        roof = {"bound": "hbm", "achieved": kb / t_dom / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": kf / t_dom / 1e12, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = counter_traffic(w.name if S == 1 else f"{w.name}_s{S}", kernel_symbol(dom, w))
    roof["traffic_ratio"] = roof["traffic"] / kb if roof["traffic"] else None
    roof["algorithmic_bytes"] = kb
    roof["algorithmic_flops"] = kf
    roof["kernel"] = dom
    roof["avg_us"] = avg_us[dom]

    step_s = ms_per_step * 1e-3
    bound_s = max(total_bytes / (PEAK_HBM_GBS * 1e9), total_flops / (PEAK_BF16_TFLOPS * 1e12))
    res = {
        "value": B * S * steps / elapsed,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_per_step,
        "dtype": dtype_of(w),
        "config": {
            "workload": w.name + (f"_s{S}" if S > 1 else ""), "batch": B, "query_tokens": S,
            "heads": H, "max_seq_len": w.max_seq_len,
            "kv_cache": "fp8_e4m3_block128" if w.fp8 else "bf16",
            "selection": (f"top-{k}" if k else ("ragged U{%d..%d}" % w.ragged if w.ragged else "dense")),
            "rows_per_step": n_rows, "replicas": R,
            "launch": "eager" if args.eager else f"hip graph replay, {G} steps per graph",
            "entry": "mla_decode_step" if FUSED else "mla_cache_write + mla_decode",
        },
        "latent_cache_gbps": n_rows * row_bytes / step_s / 1e9,
        "step_algorithmic_bytes": total_bytes,
        "step_algorithmic_flops": total_flops,
        "step_hbm_gbps": total_bytes / step_s / 1e9,
        "step_hbm_frac": total_bytes / step_s / 1e9 / PEAK_HBM_GBS,
        "step_mfma_frac": total_flops / step_s / 1e12 / PEAK_BF16_TFLOPS,
        "step_roofline_frac": bound_s / step_s,
        "step_bound": "hbm" if total_bytes / (PEAK_HBM_GBS * 1e9) >= total_flops / (PEAK_BF16_TFLOPS * 1e12)
        else "mfma",
        "kernel_avg_us": avg_us,
        "roofline": roof,
    }
    return res, x


def measure_oproj(w, x, steps, warmup, mla, synth, torch, np):
    """The step after the decode path, both ways the MLA article gives it, on
    workload w's inputs (s = 1): (a) mla_decode (with its up-projection) then
    mla_output_projection with W_O [d_model][H * 128]; (b) mla_decode_latent
    then mla_output_projection with the offline-fused W_OV = W_O W_UV
    [d_model][H * 512].  Each path is captured in a HIP graph and `steps`
    replays are timed; the projection kernels are also timed alone with
    dispatch-stamped events."""
    dev = "cuda:0"
    B, H, T = w.batch, w.heads, w.max_seq_len
    D = synth.D_MODEL
    w_o = synth.make_w_o(H, D, seed=w.seed + 500).to(dev)
    wkv_b = x["wkv_b"].to(dev)
    w_ov = torch.empty(D, H * 512, dtype=torch.bfloat16, device=dev)
    for h in range(H):  # fp32 products of the bf16 weights, rounded once (setup, not timed)
        w_ov[:, 512 * h:512 * h + 512] = (w_o[:, 128 * h:128 * h + 128].float()
                                          @ wkv_b[h, 128:, :].float()).to(torch.bfloat16)
    if w.fp8:
        kv = torch.zeros(B, T, 512, dtype=torch.uint8, device=dev)
        sc = torch.zeros(B, T, 4, dtype=torch.float32, device=dev)
        pe = torch.zeros(B, T, 64, dtype=torch.bfloat16, device=dev)
        mla.cache_write(x["kv"].to(dev), x["pe"].to(dev), torch.zeros(B, dtype=torch.int32, device=dev),
                        kv, pe, kv_scale=sc)
    else:
        kv, sc, pe = x["kv"].to(dev), None, x["pe"].to(dev)
    qn, qp, lens = x["q_nope"].to(dev), x["q_pe"].to(dev), x["cache_lens"].to(dev)
    topk = None if x["topk_idx"] is None else x["topk_idx"].to(dev)
    p = mla.make_params(B, H, T, 1 if w.fp8 else 0, topk=w.topk)
    ws = torch.empty(mla.decode_workspace_size(p), dtype=torch.uint8, device=dev)
    out = torch.empty(B, 1, H, 128, dtype=torch.bfloat16, device=dev)
    lat = torch.empty(B, 1, H, 512, dtype=torch.bfloat16, device=dev)
    y = torch.empty(B, 1, D, dtype=torch.bfloat16, device=dev)

    def path_a(ev=None):
        mla.decode(qn, qp, wkv_b, kv, pe, lens, kv_scale=sc, topk_idx=topk, out=out, workspace=ws)
        mla.output_projection(out, w_o, mla.OPROJ_WO, y=y, trace_events=ev)

    def path_b(ev=None):
        mla.decode_latent(qn, qp, wkv_b, kv, pe, lens, kv_scale=sc, topk_idx=topk, o_lat=lat,
                          workspace=ws)
        mla.output_projection(lat, w_ov, mla.OPROJ_WOV, y=y, trace_events=ev)

    res = {"d_model": D, "w_o_bytes": w_o.numel() * 2, "w_ov_bytes": w_ov.numel() * 2,
           "workload": w.name}
    hev = HipEvents()
    for name, fn in (("w_o", path_a), ("w_ov", path_b)):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            g.replay()
        torch.cuda.synchronize()
        res[f"path_{name}_us"] = 1e6 * (time.perf_counter() - t0) / steps
        ev = hev.create(2 * steps)
        arrs = [(ctypes.c_void_p * 2)(*ev[2 * i: 2 * i + 2]) for i in range(steps)]
        torch.cuda._sleep(int(2e8))
        for i in range(steps):
            fn(ev=ctypes.addressof(arrs[i]))
        torch.cuda.synchronize()
        kus = 1e3 * float(np.mean([hev.elapsed_ms(ev[2 * i], ev[2 * i + 1]) for i in range(steps)]))
        hev.destroy(ev)
        res[f"oproj_{name}_kernel_us"] = kus
        res[f"oproj_{name}_gbps"] = res[f"{name}_bytes"] / (kus * 1e-6) / 1e9
        del g
    res["w_ov_path_over_w_o_path"] = res["path_w_ov_us"] / res["path_w_o_us"]
    del w_o, w_ov, kv, sc, pe, ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--extra", default=",".join(EXTRA),
                    help="comma-separated workloads timed after the headline one ('' for none); "
                         "name:H:s runs a workload with H heads and s query tokens per sequence")
    ap.add_argument("--extra-steps", type=int, default=300)
    ap.add_argument("--extra-warmup", type=int, default=100)
    ap.add_argument("--replicas", type=int, default=0, help="0: enough to exceed the MALL")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="time eager launches, not graph replay")
    ap.add_argument("--graph-steps", type=int, default=0,
                    help="steps captured per HIP graph (0: the largest divisor of the step count up to 16)")
    ap.add_argument("--seqlen-q", type=int, default=1,
                    help="query tokens per sequence (the last s cached positions; token i sees "
                         "the rows up to its own)")
    ap.add_argument("--heads", type=int, default=0,
                    help="query heads instead of the workload's (e.g. 16: one GPU's share of 128 "
                         "heads on 8); names the workload <name>_h<heads>")
    ap.add_argument("--unfused", action="store_true",
                    help="mla_cache_write then mla_decode instead of mla_decode_step")
    ap.add_argument("--no-stream-probe", action="store_true",
                    help="skip the read-only measurement of attainable HBM bandwidth")
    ap.add_argument("--no-oproj", action="store_true",
                    help="skip the output-projection comparison (W_O after the up-projection "
                         "against the fused W_OV on the latent output)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run 5 plain device copies of BYTES bytes (reference for the "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    global FUSED
    FUSED = not args.unfused
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the decode path runs on one GPU; see the sharding notes)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        n = args.copy_calibration // 16 * 16
        src = torch.ones(n // 4, dtype=torch.int32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 5}), flush=True)
        return

    from mla_latent_kv_08_amd import mla, synth

    w = synth.WORKLOADS[args.workload]
    if args.heads and args.heads != w.heads:
        w = synth.scaled(w, heads=args.heads, name=f"{w.name}_h{args.heads}")
    S = args.seqlen_q
    print(f"bench: {w.name} s={S}: {args.warmup} warmup + {args.steps} timed steps", file=sys.stderr,
          flush=True)
    head, x = measure(w, args, args.steps, args.warmup, mla, synth, torch, np, S)
    configs = {}
    for spec in [n for n in args.extra.split(",") if n and n != args.workload]:
        we, Se = extra_workload(spec, synth, S)
        print(f"bench: {we.name} s={Se}: {args.extra_warmup} warmup + {args.extra_steps} timed steps",
              file=sys.stderr, flush=True)
        r, _ = measure(we, args, args.extra_steps, args.extra_warmup, mla, synth, torch, np, Se)
        configs[r["config"]["workload"]] = {
            "tokens_per_s": r["value"], "ms_per_step": r["ms_per_step"], "steps": r["steps"],
            "heads": r["config"]["heads"], "query_tokens": r["config"]["query_tokens"],
            "dtype": r["dtype"], "kv_cache": r["config"]["kv_cache"],
            "selection": r["config"]["selection"], "rows_per_step": r["config"]["rows_per_step"],
            "latent_cache_gbps": r["latent_cache_gbps"], "step_hbm_frac": r["step_hbm_frac"],
            "step_mfma_frac": r["step_mfma_frac"], "step_roofline_frac": r["step_roofline_frac"],
            "step_bound": r["step_bound"], "kernel_avg_us": r["kernel_avg_us"],
            "roofline": r["roofline"],
        }
    oproj = None
    if not args.no_oproj and S == 1:
        print(f"bench: output projection of {w.name}: W_O path and fused W_OV path", file=sys.stderr,
              flush=True)
        oproj = measure_oproj(w, x, args.extra_steps, args.extra_warmup, mla, synth, torch, np)
    stream_gbps = None if args.no_stream_probe else stream_probe(torch)
    for r in [head] + list(configs.values()):
        roof = r["roofline"]
        if stream_gbps and roof["bound"] == "hbm":
            roof["frac_of_measured_read"] = roof["achieved"] / stream_gbps

    result = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic",
        "config": head["config"],
        "latent_cache_gbps": head["latent_cache_gbps"],
        "latent_cache_frac": head["latent_cache_gbps"] / PEAK_HBM_GBS,
        "step_hbm_gbps": head["step_hbm_gbps"],
        "step_hbm_frac": head["step_hbm_frac"],
        "step_mfma_frac": head["step_mfma_frac"],
        "step_roofline_frac": head["step_roofline_frac"],
        "step_bound": head["step_bound"],
        "hbm_read_gbps": stream_gbps,
        "hbm_read_probe": "read-only streaming kernel over 2 GiB, 16-byte non-temporal loads",
        "kernel_avg_us": head["kernel_avg_us"],
        "kernel_timing": "dispatch-stamped HIP events, eager pass of the same K steps",
        "roofline": head["roofline"],
        "configs": configs,
        "output_projection": oproj,
    }
    if not args.no_cpu_baseline:
        import oracle
        result["cpu_baseline"] = cpu_baseline(w, x, args.cpu_seconds, oracle, synth, np, torch)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
