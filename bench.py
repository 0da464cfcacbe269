"""Throughput of the DSA lightning-indexer path on one MI355X.

A step is the whole hot path for one batch: one F layer of the IndexCache
stack (idx_indexcache_layer), which quantises + scatters this step's new K
rows, scores every causal position and selects the top-k into the persistent
buffer (on decode batches over long contexts the scores never leave the chip:
fused score + top-k).  Inputs are resident in HBM before timing starts.

The headline workload is the 128K decode batch (8 requests x 131072
positions, k = 2048).  The JSON line also carries every other workload:

  prefill-24k+8k     chunked prefill, 24576 cached + 8192 new tokens
  decode-64x16k-32k  64 decode requests, contexts uniform in [16K, 32K]
  prefill-1k         T = S = 1024 causal, k = 256
  stack-16L-32x64k   16 layers, FSSS x4, 32 decode requests at 64K (a step is
                     the whole stack; all-F, and FSSS with the index group's
                     physical rows converted after each F layer, are timed
                     beside it)
  decode-8x128k-fp4  the headline batch over the FP4 indexer K cache (a step:
                     idx_indexcache_layer_fp4, the same F layer)

each with its step time, throughput, the step's per-kernel times and the
dominant kernel's roofline.  Per-kernel times come from a separate traced loop
(idx_trace_begin: HIP events on the kernels' stream around every launch), so
the timed loop that gives `value` carries no extra events.  Algorithmic work
per launch of the dominant kernel:

  decode scoring   sum_t (p_t + 1) * 132 B of K + per token 8192 B of q,
                   256 B of weights, 256 + 132 B of its new K row
  FP4 decode       sum_t (p_t + 1) * 68 B of K + per token 8192 B of q,
                   256 B of weights, 256 + 68 B of its new K row
  prefill scoring  2 * 64 * 128 * sum_t (p_t + 1) fp8 flops (causal pairs)

Decode steps rotate through several copies of the K cache so the 256 MB
Infinity Cache cannot serve the K bytes across iterations.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-next-rows]
    python bench.py --copy-calibration     # plain 1 GiB copies, for the counter scale

`roofline.traffic` is the dominant kernel's HBM bytes per launch as the
FETCH_SIZE / WRITE_SIZE counters saw them in a profiled run of this script,
scaled by what the same counters read for a plain copy of known size.  It is
read from the committed counter summary and reported only while the kernel's
sources are the ones that summary was taken on (else null).
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "indexer query-tokens/s (128K decode, 32K prefill); % of HBM / fp8 MFMA roof"
HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0
PROFILES = os.path.join(ROOT, "profiles")
CSRC = "sparse_attention_token_fp8_amd/csrc/"
HEADLINE = "decode-8x128k"
SINGLE_LAYER = ("decode-8x128k", "prefill-24k+8k", "decode-64x16k-32k", "prefill-1k",
                "decode-8x128k-fp4")
FP4_SUFFIX = "-fp4"
STACK = "stack-16L-32x64k"
# sources whose code the dominant kernels are built from (for the traffic digest)
KERNEL_SOURCES = {
    "score_keep_kernel": ("fused.hip", "score_device.hpp", "fp4_device.hpp", "topk_device.hpp",
                          "common.hpp", "quant_device.hpp"),
    "score_prefill_kernel": ("score.hip", "score_device.hpp", "common.hpp", "quant_device.hpp"),
    "score_fp4_decode_kernel": ("fp4.hip", "fp4_device.hpp", "score_device.hpp", "common.hpp",
                                "quant_device.hpp"),
    "score_keep_fp4_kernel": ("fused.hip", "fp4_device.hpp", "score_device.hpp", "topk_device.hpp",
                              "common.hpp", "quant_device.hpp"),
}
DECODE_KERNELS = ("score_keep_kernel", "score_decode_write_kernel", "score_decode_kernel",
                  "score_fp4_decode_kernel", "score_keep_fp4_kernel")
FP4_KERNELS = ("score_fp4_decode_kernel", "score_fp4_prefill_kernel", "score_keep_fp4_kernel")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workloads", default=",".join(SINGLE_LAYER + (STACK,)),
                   help="comma-separated; the headline " + HEADLINE + " always runs")
    p.add_argument("--replicas", type=int, default=4)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-next-rows", action="store_true",
                   help="skip the q-fold / physical-conversion / mixed-batch / graph measurements")
    p.add_argument("--cpu-tokens", type=int, default=8, help="query tokens the oracle scores per pass")
    p.add_argument("--cpu-seconds", type=float, default=5.0, help="minimum timed oracle work per workload")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run plain 1 GiB device copies (counter calibration)")
    return p.parse_args()


def build_flags(src):
    """The hipcc flags a source is compiled with (read from build.py by path)."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_idx_build_flags", os.path.join(ROOT, "sparse_attention_token_fp8_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return [os.path.basename(f) if f.startswith("-I") else f
            for f in mod.COMMON + mod.EXTRA.get(src, [])]


def _code_only(text):
    """Source text without comments and with runs of blank space collapsed, so an
    edit of comments alone keeps the digest."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def sources_digest(kernel):
    """Digest of a dominant kernel's code (comments aside) and its compile flags."""
    files = KERNEL_SOURCES[kernel]
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, CSRC, f)) as fh:
            h.update(_code_only(fh.read()).encode())
    h.update(" ".join(build_flags(files[0])).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed counter
    summary, or None when there is none or the kernel's sources have changed."""
    path = os.path.join(PROFILES, f"traffic_{kernel}_{workload}.md")
    if kernel not in KERNEL_SOURCES or not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            line = line.strip().strip("`")
            if line.startswith(("traffic_bytes_per_launch:", "sources_digest:")):
                key, val = line.split(":", 1)
                fields[key] = val.strip()
    if fields.get("sources_digest") != sources_digest(kernel):
        return None
    return int(fields["traffic_bytes_per_launch"]) if "traffic_bytes_per_launch" in fields else None


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def copy_calibration(torch, nbytes=1 << 30, launches=4):
    """Plain device-to-device copies of a known size (the counter scale)."""
    x = torch.full((nbytes // 4,), 7, dtype=torch.int32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(launches):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes,
                      "launches": launches}), flush=True)


# ------------------------------------------------------------------ setup --

def setup(m, torch, wl, replicas, layer=0, fp4=False):
    """Device state: cache replicas with the context K (FP8, or FP4), q_fp8 / w,
    new K rows."""
    import concurrent.futures as cf
    t0 = time.time()
    batch = m.Batch(wl.seq_lens, wl.query_start_loc, wl.block_table)
    kind = m.KCacheFP4 if fp4 else m.KCache
    write = m.idx_quant_write_k_fp4 if fp4 else m.idx_quant_write_k
    cache = kind(wl.num_blocks, fill=0)
    reqs = [r for r in range(wl.num_reqs) if wl.seq_lens[r] > wl.new_tokens[r]]
    nw = max(1, min(16, len(os.sched_getaffinity(0))))
    with cf.ThreadPoolExecutor(nw) as ex:
        for kb, slots in ex.map(lambda r: wl.ctx_rows(layer, [r]), reqs):
            write(torch.from_numpy(kb.view(np.int16)).cuda(), torch.from_numpy(slots).cuda(), cache)
    q8, w, _ = m.idx_quant_q_fold_w(torch.from_numpy(wl.q_bits(layer).view(np.int16)).cuda(),
                                    torch.from_numpy(wl.w_raw(layer)).cuda())
    nb, ns = wl.new_rows(layer)
    k_new = torch.from_numpy(nb.view(np.int16)).cuda()
    slots = torch.from_numpy(ns).cuda()
    caches = [cache] + [kind(wl.num_blocks, tensor=cache.tensor.clone()) for _ in range(replicas - 1)]
    torch.cuda.synchronize()
    log(f"setup {wl.name}: {time.time() - t0:.1f}s, {replicas} cache copies of "
        f"{cache.tensor.numel() / 1e6:.1f} MB")
    return dict(batch=batch, caches=caches, q8=q8, w=w, k_new=k_new, slots=slots)


def algorithmic(wl, fp4=False):
    """Per-step algorithmic work of one F layer (the measurement section's counts):
    decode scoring bytes (K of every causal position, q, w, the new K row; for
    the FP4 cache 68 B per position and the new rows outside the scoring
    launch), the step's bytes (plus the top-k indices written) and the MFMA
    flops of the causal (token, position) pairs."""
    P = int(np.sum(wl.token_pos() + 1))
    T = wl.num_tokens
    if fp4:
        score_bytes = P * 68 + T * (64 * 128 + 64 * 4 + 256 + 68)
        step_bytes = score_bytes + T * 4 * wl.k
    else:
        score_bytes = P * 132 + T * (64 * 128 + 64 * 4 + 256 + 132)
        step_bytes = score_bytes + T * 4 * wl.k
    flops = 2 * 64 * 128 * P
    return dict(positions=P, score_bytes=score_bytes, step_bytes=step_bytes, flops=flops)


def time_loop(torch, fn, steps, warmup):
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        fn(i)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps   # ms


def step_quantiles(m, torch, fn, steps, warmup):
    """p10 / median / p90 of single steps, each bracketed by its own timing events
    (device-scope release) on the current stream; a separate loop from the mean,
    which uses one event pair."""
    for i in range(warmup):
        fn(i)
    ev = [(m.HipEvent(), m.HipEvent()) for _ in range(steps)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(ev):
        a.record()
        fn(i)
        b.record()
    torch.cuda.synchronize()
    t = np.sort(np.array([a.elapsed_ms(b) for a, b in ev]))
    q = lambda f: round(float(t[min(len(t) - 1, int(f * (len(t) - 1) + 0.5))]), 5)
    return {"p10": q(0.1), "p50": q(0.5), "p90": q(0.9), "steps": steps}


def kernel_times(m, torch, fn, steps, warmup):
    """Average time of each kernel the step launches, from a traced loop (the
    library's idx_trace_begin: HIP events recorded on the kernels' stream
    around every launch, recorded with a device-scope release so that they add
    next to nothing to the kernels they bracket).  Returns {name: (mean ms,
    launches)} in launch order."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    with m.KernelTrace(capacity=64 * steps) as tr:
        for i in range(steps):
            fn(i)
    acc = {}
    for name, ms in tr.kernels:
        s, n = acc.get(name, (0.0, 0))
        acc[name] = (s + ms, n + 1)
    return {name: (s / n, n) for name, (s, n) in acc.items()}


def dominant(kernels):
    """The kernel that takes the most of the step's time in a trace."""
    return max(kernels, key=lambda n: kernels[n][0] * kernels[n][1])


def roofline(wl, name, kernel, ms, launches):
    """Roofline entry of the dominant kernel from its measured time per launch."""
    a = algorithmic(wl, fp4=kernel in FP4_KERNELS)
    if kernel in DECODE_KERNELS:
        ach = a["score_bytes"] / (ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": measured_traffic(kernel, name),
                "kernel": kernel, "ms_per_launch": round(ms, 5), "launches_per_step": launches,
                "bytes_per_launch": a["score_bytes"]}
    ach = a["flops"] / (ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": round(ach, 1), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(ach / FP8_PEAK_TFLOPS, 4), "traffic": measured_traffic(kernel, name),
            "kernel": kernel, "ms_per_launch": round(ms, 5), "launches_per_step": launches,
            "flops_per_launch": a["flops"]}


def dominant_ms(m, torch, kernel, d, wl, reps, ws, steps, warmup):
    """Time per launch of the step's dominant kernel, launched back to back on its
    own through the entry point that runs exactly that launch: the fused
    path's scoring (idx_score_candidates with the step's new K rows) or the
    prefill scoring (idx_logits).  Events bracket the whole loop, so the
    per-launch time carries one launch gap and no event overhead."""
    B, k = d["batch"], wl.k
    if kernel in ("score_keep_kernel", "score_keep_fp4_kernel"):
        cand = m.idx_score_candidates if kernel == "score_keep_kernel" else m.idx_score_candidates_fp4
        fn = lambda i: cand(d["q8"], d["w"], d["caches"][i % reps], B, k, ws, d["k_new"], d["slots"])
    elif kernel in ("score_prefill_kernel",) + FP4_KERNELS:
        logits = torch.empty((wl.num_tokens, wl.max_seq_len), dtype=torch.float32, device="cuda")
        score = m.idx_logits if kernel == "score_prefill_kernel" else m.idx_logits_fp4
        fn = lambda i: score(d["q8"], d["w"], d["caches"][i % reps], B, logits=logits)
    else:
        return None
    return time_loop(torch, fn, steps, warmup)


def config_of(wl, reps, fp4=False):
    return {"workload": wl.name + (FP4_SUFFIX if fp4 else ""), "requests": wl.num_reqs,
            "query_tokens": wl.num_tokens, "max_context": wl.max_seq_len, "index_topk": wl.k,
            "heads": 64, "head_dim": 128, "block_size": 64, "layers": wl.num_layers,
            "cache_copies": reps, "k_cache": "fp4 e2m1 + e8m0 per 32" if fp4 else "fp8 e4m3 + fp32"}


def run_workload(m, torch, name, args):
    from synth import CONFIGS, make_workload
    fp4 = name.endswith(FP4_SUFFIX)
    wl = make_workload(CONFIGS[name[:-len(FP4_SUFFIX)] if fp4 else name])
    decode = wl.max_query_len == 1
    reps = args.replicas if decode else 1
    d = setup(m, torch, wl, reps, fp4=fp4)
    B, k = d["batch"], wl.k
    topk = torch.empty((wl.num_tokens, k), dtype=torch.int32, device="cuda")
    wsize = m.idx_score_topk_fp4_workspace_size(B, k) if fp4 else m.idx_score_topk_workspace_size(B, k)
    ws = torch.empty(max(256, wsize), dtype=torch.uint8, device="cuda")

    def step(i):                                       # one F layer: new K rows, scores, top-k
        c = d["caches"][i % reps]
        if fp4:
            m.idx_indexcache_layer_fp4(d["k_new"], c, d["q8"], d["w"], True, True, d["slots"], B, k,
                                       topk, workspace=ws)
        else:
            m.idx_indexcache_layer(d["k_new"], c, d["q8"], d["w"], True, True, d["slots"], B, k,
                                   topk, workspace=ws)

    ms_step = time_loop(torch, step, args.steps, args.warmup)
    quant = step_quantiles(m, torch, step, max(args.steps, 50), args.warmup)
    kern = kernel_times(m, torch, step, min(args.steps, 20), 2)
    dom = dominant(kern)
    ms_dom = dominant_ms(m, torch, dom, d, wl, reps, ws, args.steps, args.warmup)
    roof = roofline(wl, name, dom, ms_dom if ms_dom is not None else kern[dom][0], kern[dom][1])
    a = algorithmic(wl, fp4=fp4)
    res = dict(workload=name, value=round(wl.num_tokens / (ms_step * 1e-3), 1),
               ms_per_step=round(ms_step, 5), step_ms_quantiles=quant, roofline=roof,
               kernels_ms={n: round(v[0], 5) for n, v in kern.items()},
               step_hbm_frac=round(a["step_bytes"] / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
               step_mfma_frac=round(a["flops"] / (ms_step * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 4),
               config=config_of(wl, reps, fp4))
    log(f"{name}: {ms_step * 1e3:.1f} us/step; " +
        ", ".join(f"{n} {v[0] * 1e3:.1f} us" for n, v in kern.items()) +
        f"; {roof['kernel']} alone {roof['ms_per_launch'] * 1e3:.1f} us, "
        f"{roof['frac'] * 100:.1f}% of {roof['bound']} peak")
    del d, topk, ws
    torch.cuda.empty_cache()
    wl.fp4 = fp4
    return res, wl


def run_stack(m, torch, args):
    """stack-16L-32x64k: the 16-layer stack (idx_indexcache_stack) with the FSSS x4
    schedule, the step, and with every layer F beside it.  Layer 0's context K
    is written once and copied into 16 distinct caches, so every F layer reads
    its own 277 MB."""
    import concurrent.futures as cf
    from synth import CONFIGS, make_workload
    t0 = time.time()
    wl = make_workload(CONFIGS[STACK])
    batch = m.Batch(wl.seq_lens, wl.query_start_loc, wl.block_table)
    cache = m.KCache(wl.num_blocks, fill=0)
    nw = max(1, min(16, len(os.sched_getaffinity(0))))
    with cf.ThreadPoolExecutor(nw) as ex:
        for kb, slots in ex.map(lambda r: wl.ctx_rows(0, [r]), range(wl.num_reqs)):
            m.idx_quant_write_k(torch.from_numpy(kb.view(np.int16)).cuda(),
                                torch.from_numpy(slots).cuda(), cache)
    layers = []
    for l in range(wl.num_layers):
        c = cache if l == 0 else m.KCache(wl.num_blocks, tensor=cache.tensor.clone())
        q8, w, _ = m.idx_quant_q_fold_w(torch.from_numpy(wl.q_bits(l).view(np.int16)).cuda(),
                                        torch.from_numpy(wl.w_raw(l)).cuda())
        nb, ns = wl.new_rows(l)
        layers.append((torch.from_numpy(nb.view(np.int16)).cuda(), c, q8, w))
    slots = torch.from_numpy(ns).cuda()
    topk = torch.empty((wl.num_tokens, wl.k), dtype=torch.int32, device="cuda")
    ws = torch.empty(m.idx_score_topk_workspace_size(batch, wl.k), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    log(f"setup {wl.name}: {time.time() - t0:.1f}s, {wl.num_layers} caches")
    fsss = m.idx_layer_schedule(True, wl.pattern, 1, 2, wl.num_layers)

    def stack(full):
        return lambda i: m.idx_indexcache_stack(layers, full, True, slots, batch, wl.k, topk,
                                                workspace=ws)

    # the index group's physical rows (block size 64), converted once after each F layer
    phys = m.Physical(wl.num_tokens, wl.k, wl.num_blocks)

    def stack_physical(i):
        m.idx_indexcache_stack_physical(layers, fsss, True, slots, batch, wl.k, topk, phys,
                                        workspace=ws)

    steps = max(5, args.steps // 2)
    ms_fsss = time_loop(torch, stack(fsss), steps, 3)
    ms_all_f = time_loop(torch, stack([True] * wl.num_layers), steps, 3)
    ms_phys = time_loop(torch, stack_physical, steps, 3)
    quant = step_quantiles(m, torch, stack(fsss), max(steps, 20), 3)
    kern = kernel_times(m, torch, stack(fsss), 5, 1)
    kern = {n: (ms, cnt // 5) for n, (ms, cnt) in kern.items()}   # launches per stack
    dom = dominant(kern)
    f_layers = [l for l, f in enumerate(fsss) if f]
    dom_state = {"batch": batch, "caches": [layers[l][1] for l in f_layers],
                 "q8": layers[0][2], "w": layers[0][3], "k_new": layers[0][0], "slots": slots}
    ms_dom = dominant_ms(m, torch, dom, dom_state, wl, len(f_layers), ws, steps, 3)
    roof = roofline(wl, STACK, dom, ms_dom if ms_dom is not None else kern[dom][0], kern[dom][1])
    log(f"{wl.name}: FSSS x4 {ms_fsss * 1e3:.1f} us, all F {ms_all_f * 1e3:.1f} us per stack; " +
        ", ".join(f"{n} {v[0] * 1e3:.1f} us x{v[1]}" for n, v in kern.items()))
    res = {"workload": wl.name, "value": round(wl.num_tokens / (ms_fsss * 1e-3), 1),
           "ms_per_step": round(ms_fsss, 5), "step_ms_quantiles": quant, "roofline": roof,
           "kernels_ms": {n: round(v[0], 5) for n, v in kern.items()},
           "kernel_launches_per_step": {n: v[1] for n, v in kern.items()},
           "f_layers": [i for i, f in enumerate(fsss) if f], "ms_all_f": round(ms_all_f, 5),
           "ms_fsss_with_physical_rows": round(ms_phys, 5),
           "all_f_over_fsss": round(ms_all_f / ms_fsss, 3), "config": config_of(wl, 1)}
    del layers, cache, topk, ws, phys
    torch.cuda.empty_cache()
    return res, wl


def _layers(m, torch, wl):
    """Per-layer device state for a multi-layer workload (context K, q_fp8 / w, new K rows)."""
    layers = []
    reqs = [r for r in range(wl.num_reqs) if wl.seq_lens[r] > wl.new_tokens[r]]
    for l in range(wl.num_layers):
        cache = m.KCache(wl.num_blocks, fill=0)
        for r in reqs:
            kb, slots = wl.ctx_rows(l, [r])
            m.idx_quant_write_k(torch.from_numpy(kb.view(np.int16)).cuda(),
                                torch.from_numpy(slots).cuda(), cache)
        q8, w, _ = m.idx_quant_q_fold_w(torch.from_numpy(wl.q_bits(l).view(np.int16)).cuda(),
                                        torch.from_numpy(wl.w_raw(l)).cuda())
        nb, ns = wl.new_rows(l)
        layers.append((torch.from_numpy(nb.view(np.int16)).cuda(), cache, q8, w))
    return layers, torch.from_numpy(ns).cuda()


def run_next_rows(m, torch, steps=20, warmup=3):
    """The steps next to the path, each timed live with HIP events:
    NEXT-1 q quantisation + weight fold and NEXT-2 logical -> physical top-k on
    the 32K prefill chunk's shapes (HBM-bound, inputs rotated over three copies
    so the Infinity Cache cannot serve them); NEXT-3 a mixed decode + prefill
    batch in one launch against the two launches it replaces, and a 16-layer
    FSSS x4 stack of small decode layers replayed from a HIP graph against
    eager launches."""
    from synth import CONFIGS, make_workload, random_batch
    out = {}
    wl = make_workload(CONFIGS["prefill-24k+8k"])
    T, H, D, k = wl.num_tokens, 64, 128, wl.k
    g = torch.Generator(device="cuda")
    g.manual_seed(20251)

    # NEXT-1
    qs = [torch.randn((T, H, D), generator=g, device="cuda").to(torch.bfloat16) for _ in range(3)]
    wr = [torch.randn((T, H), generator=g, device="cuda") for _ in range(3)]
    q8 = [torch.empty((T, H, D), dtype=torch.uint8, device="cuda") for _ in range(3)]
    wf = [torch.empty((T, H), dtype=torch.float32, device="cuda") for _ in range(3)]
    sc = [torch.empty((T, H), dtype=torch.float32, device="cuda") for _ in range(3)]
    ms = time_loop(torch, lambda i: m.idx_quant_q_fold_w(qs[i % 3], wr[i % 3], q_fp8=q8[i % 3],
                                                         w_folded=wf[i % 3], q_scale=sc[i % 3]),
                   steps, warmup)
    nbytes = T * H * (2 * D + 4) + T * H * (D + 4 + 4)
    out["next1_quant_q_fold"] = _hbm_row("quant_q_fold_kernel", nbytes, ms, f"{T} tokens x {H} heads")
    del qs, wr, q8, wf, sc

    # NEXT-2
    batch = m.Batch(wl.seq_lens, wl.query_start_loc, wl.block_table)
    hi = torch.from_numpy((wl.token_pos() + 1).astype(np.float32)).cuda()[:, None]
    lg = [torch.sort((torch.rand((T, k), generator=g, device="cuda") * hi).to(torch.int32), dim=1)[0]
          for _ in range(3)]
    ph = [torch.empty((T, k), dtype=torch.int32, device="cuda") for _ in range(3)]
    vc = [torch.empty((T,), dtype=torch.int32, device="cuda") for _ in range(3)]
    ms = time_loop(torch, lambda i: m.idx_topk_to_physical(lg[i % 3], batch, wl.num_blocks,
                                                           physical=ph[i % 3], valid_counts=vc[i % 3]),
                   steps, warmup)
    nbytes = 2 * T * k * 4 + T * 4
    out["next2_topk_to_physical"] = _hbm_row("to_physical_kernel", nbytes, ms, f"{T} rows x k {k}")
    del lg, ph, vc

    # NEXT-3: one mixed launch (64 decode tokens, then a 2048-token prefill chunk)
    rng = np.random.default_rng(20252)
    dec = rng.integers(16384, 32769, 64).tolist()
    mw = random_batch(20252, dec + [16384 + 2048], [1] * 64 + [2048], k=2048)
    d = setup(m, torch, mw, 1)
    cache = d["caches"][0]
    mixed = m.Batch(mw.seq_lens, mw.query_start_loc, mw.block_table, num_decode_tokens=64)
    bd = m.Batch(mw.seq_lens[:64], mw.query_start_loc[:65], mw.block_table[:64])
    bp = m.Batch(mw.seq_lens[64:], mw.query_start_loc[64:] - 64, mw.block_table[64:])
    lm = torch.empty((mw.num_tokens, mw.max_seq_len), dtype=torch.float32, device="cuda")
    ld = torch.empty((64, bd.max_seq_len), dtype=torch.float32, device="cuda")
    lp = torch.empty((2048, bp.max_seq_len), dtype=torch.float32, device="cuda")
    q8d, wd, q8p, wp = d["q8"][:64], d["w"][:64], d["q8"][64:], d["w"][64:]
    def one(i):
        m.idx_logits(d["q8"], d["w"], cache, mixed, logits=lm)

    def two(i):
        m.idx_logits(q8d, wd, cache, bd, logits=ld)
        m.idx_logits(q8p, wp, cache, bp, logits=lp)

    # alternated (one, two, one, two), each the better of its two runs, so neither
    # form is timed alone right after the setup
    r1, r2 = [], []
    for _ in range(2):
        r1.append(time_loop(torch, one, steps, warmup))
        r2.append(time_loop(torch, two, steps, warmup))
    ms1, ms2 = min(r1), min(r2)
    a = algorithmic(mw)
    pos = mw.token_pos() + 1
    dec_bytes = int(np.sum(pos[:64])) * 132 + 64 * (H * D + H * 4)
    pre_flops = 2 * H * D * int(np.sum(pos[64:]))
    bound_ms = max(dec_bytes / (HBM_PEAK_GBS * 1e9), pre_flops / (FP8_PEAK_TFLOPS * 1e12)) * 1e3
    out["next3_mixed_batch"] = {
        "kernel": "score_mixed_kernel (idx_logits, num_decode_tokens = 64)",
        "batch": "64 decode tokens over 16K-32K contexts + one 2048-token prefill chunk over 16K",
        "ms_one_launch": round(ms1, 5), "ms_two_launches": round(ms2, 5),
        "decode_bytes": dec_bytes, "prefill_flops": pre_flops, "positions": a["positions"],
        "bound": "max(hbm, mfma)", "bound_ms": round(bound_ms, 5), "frac": round(bound_ms / ms1, 4)}
    del d, cache, lm, ld, lp
    torch.cuda.empty_cache()

    # NEXT-3: the F/S stack from a HIP graph
    sw = random_batch(20253, [4096] * 8, 1, k=512, num_layers=16, pattern="FSSS" * 4)
    layers, slots = _layers(m, torch, sw)
    sb = m.Batch(sw.seq_lens, sw.query_start_loc, sw.block_table)
    full = m.idx_layer_schedule(True, sw.pattern, 1, 2, sw.num_layers)
    topk = torch.empty((sw.num_tokens, sw.k), dtype=torch.int32, device="cuda")
    ws = torch.empty(m.idx_score_topk_workspace_size(sb, sw.k), dtype=torch.uint8, device="cuda")

    def stack(i):
        m.idx_indexcache_stack(layers, full, True, slots, sb, sw.k, topk, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        stack(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        stack(0)
    # alternated (eager, graph, eager, graph), each the better of its two runs
    re, rg = [], []
    for _ in range(2):
        re.append(time_loop(torch, stack, steps, warmup))
        rg.append(time_loop(torch, lambda i: graph.replay(), steps, warmup))
    ms_eager, ms_graph = min(re), min(rg)
    out["next3_stack_graph"] = {
        "stack": "16 layers FSSS x4, 8 decode requests x 4096 positions, k 512",
        "ms_eager": round(ms_eager, 5), "ms_graph_replay": round(ms_graph, 5),
        "speedup": round(ms_eager / ms_graph, 3)}
    del graph, layers
    torch.cuda.empty_cache()
    return out




def _hbm_row(kernel, nbytes, ms, shape):
    ach = nbytes / (ms * 1e-3) / 1e9
    return {"kernel": kernel, "shape": shape, "bound": "hbm", "bytes_per_launch": nbytes,
            "ms_per_launch": round(ms, 5), "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4)}


def cpu_baseline(wl, sample, min_seconds=5.0):
    """The oracle, as it stands, on `sample` query tokens of the workload (their
    requests' new K rows written into each layer's cache, fp64 scores over the
    full causal range, full-sort top-k on the F layers), repeated until at least
    `min_seconds` of work has been timed.  Returns query-tokens/s of that work."""
    import concurrent.futures as cf
    import oracle
    from oracle import fp4cache, logits as olog, quant as oquant, topk as otopk
    fp4 = getattr(wl, "fp4", False)
    write = fp4cache.quant_write_k if fp4 else oquant.quant_write_k
    score_row = fp4cache.logits_row if fp4 else olog.logits_row
    new_cache = ((lambda: fp4cache.new_cache(wl.num_blocks)) if fp4 else
                 (lambda: np.zeros((wl.num_blocks, 64, 132), np.uint8)))
    try:
        from threadpoolctl import threadpool_info
        blas = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        blas = None
    tokens = np.unique(np.linspace(0, wl.num_tokens - 1, min(sample, wl.num_tokens)).astype(int))
    reqs = sorted(set(int(r) for r in wl.token_req()[tokens]))
    full = [c == "F" for c in wl.pattern] if wl.num_layers > 1 else [True]
    ob = oracle.Batch(wl.seq_lens, wl.query_start_loc, wl.block_table)
    nw = max(1, min(16, len(os.sched_getaffinity(0))))
    layers = []
    for layer, is_f in enumerate(full):                 # setup, not timed
        cache = new_cache()
        new = {}

        def ctx(r, layer=layer, cache=cache, is_f=is_f):
            kb = wl.request_k(layer, r)
            L, n = int(wl.seq_lens[r]), int(wl.new_tokens[r])
            if is_f:                                    # S layers score nothing: no context needed
                write(cache, kb[:L - n], wl.slots(r, np.arange(L - n)))
            return r, (kb[L - n:], wl.slots(r, np.arange(L - n, L)))

        with cf.ThreadPoolExecutor(nw) as ex:
            new = dict(ex.map(ctx, reqs))
        q8 = w = None
        if is_f:
            q8, qs = oquant.quantize_q(wl.q_bits(layer))
            w = oquant.fold_weights(wl.w_raw(layer), qs)
        layers.append((is_f, cache, new, q8, w))
    passes = 0
    t0 = time.time()
    while passes == 0 or time.time() - t0 < min_seconds:
        for is_f, cache, new, q8, w in layers:
            for r in reqs:                              # this step's K rows of the sampled requests
                write(cache, *new[r])
            if is_f:
                for t in tokens:
                    r, p = ob.token_request(int(t)), ob.token_position(int(t))
                    s = score_row(q8[t], w[t], cache, wl.block_table[r], p)
                    otopk.topk_row(s, wl.k)
        passes += 1
    dt = time.time() - t0
    return {"value": round(passes * len(tokens) / dt, 3), "unit": "query-tokens/s",
            "cores": len(os.sched_getaffinity(0)), "blas_threads": blas, "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": f"{passes} pass(es) over {len(tokens)} of the {wl.num_tokens} query tokens of "
                      f"{wl.name}{FP4_SUFFIX if fp4 else ''} ({wl.num_layers} layer(s): their new K "
                      f"rows{' (FP4 cache)' if fp4 else ''}, fp64 scores over the "
                      f"full causal range and a full-sort top-{wl.k} on F layers); {dt:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the library has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)
    import torch
    import sparse_attention_token_fp8_amd as m
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(torch)
        return
    names = [HEADLINE] + [n for n in args.workloads.split(",") if n and n != HEADLINE]
    results, wls = {}, {}
    for name in names:
        if name == STACK:
            results[name], wls[name] = run_stack(m, torch, args)
        else:
            results[name], wls[name] = run_workload(m, torch, name, args)
    head = results[HEADLINE]
    out = {"metric": METRIC, "value": head["value"], "unit": "query-tokens/s",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": head["ms_per_step"], "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "fp8e4m3", "data": "synthetic",
           "config": head["config"], "roofline": head["roofline"],
           "step_ms_quantiles": head["step_ms_quantiles"], "kernels_ms": head["kernels_ms"],
           "step_hbm_frac": head["step_hbm_frac"],
           "workloads": {n: r for n, r in results.items() if n != HEADLINE}}
    if not args.no_next_rows:
        try:
            out["next_rows"] = run_next_rows(m, torch)
        except Exception as e:                         # reported, never fatal to the bench line
            out["next_rows"] = {"error": f"{type(e).__name__}: {e}"}
    if not args.no_cpu_baseline:
        for name in names:
            t0 = time.time()
            cb = cpu_baseline(wls[name], args.cpu_tokens if name != STACK else 2, args.cpu_seconds)
            log(f"cpu baseline {name}: {cb['value']} query-tokens/s ({time.time() - t0:.1f} s)")
            if name == HEADLINE:
                out["cpu_baseline"] = cb
            else:
                out["workloads"][name]["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
