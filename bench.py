"""Throughput of the DSA lightning-indexer path on one MI355X.

A step is the whole hot path for one batch: one F layer of the IndexCache
stack (idx_indexcache_layer), which quantises + scatters this step's new K
rows, scores every causal position and selects the top-k into the persistent
buffer.  Inputs are resident in HBM before timing starts.  The headline workload is the 128K decode batch
(8 requests x 131072 positions, k = 2048); the 32K chunked prefill (24576
cached + 8192 new tokens) is reported alongside in the same JSON line.

Decode steps rotate through several copies of the K cache so the 256 MB
Infinity Cache cannot serve the K bytes across iterations.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
    python bench.py --copy-calibration     # plain 1 GiB copies, for the counter scale

`roofline.traffic` is the dominant kernel's HBM bytes per launch as the
FETCH_SIZE / WRITE_SIZE counters saw them in a profiled run of this script,
scaled by what the same counters read for a plain copy of known size.  It is
read from the committed counter summary and reported only while the scoring
sources are byte-identical to the ones that summary was taken on (else null).
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

METRIC = "indexer query-tokens/s (128K decode, 32K prefill); % of HBM / fp8 MFMA roof"
HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0
PROFILES = os.path.join(ROOT, "profiles")
SCORE_SOURCES = ("sparse_attention_token_fp8_amd/csrc/score.hip",
                 "sparse_attention_token_fp8_amd/csrc/common.hpp",
                 "sparse_attention_token_fp8_amd/build.py")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="decode-8x128k")
    p.add_argument("--secondary", default="prefill-24k+8k", help="'' to skip")
    p.add_argument("--replicas", type=int, default=4)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample", type=int, default=8, help="query tokens the oracle scores")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="minimum timed oracle work")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run plain 1 GiB device copies (counter calibration)")
    return p.parse_args()


def sources_digest():
    """Digest of the scoring kernels' sources and build flags."""
    h = hashlib.sha256()
    for f in SCORE_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed counter
    summary, or None when there is none or the sources have changed since."""
    path = os.path.join(PROFILES, f"traffic_{kernel}_{workload}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            line = line.strip().strip("`")
            if line.startswith(("traffic_bytes_per_launch:", "sources_digest:")):
                key, val = line.split(":", 1)
                fields[key] = val.strip()
    if fields.get("sources_digest") != sources_digest():
        return None
    return int(fields["traffic_bytes_per_launch"]) if "traffic_bytes_per_launch" in fields else None


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

def setup(m, torch, wl, replicas):
    """Device state: cache replicas with the context K, q_fp8 / w, new K rows."""
    import concurrent.futures as cf
    t0 = time.time()
    batch = m.Batch(wl.seq_lens, wl.query_start_loc, wl.block_table)
    cache = m.KCache(wl.num_blocks, fill=0)
    reqs = [r for r in range(wl.num_reqs) if wl.seq_lens[r] > wl.new_tokens[r]]
    nw = max(1, min(16, len(os.sched_getaffinity(0))))
    with cf.ThreadPoolExecutor(nw) as ex:
        for kb, slots in ex.map(lambda r: wl.ctx_rows(0, [r]), reqs):
            m.idx_quant_write_k(torch.from_numpy(kb.view(np.int16)).cuda(),
                                torch.from_numpy(slots).cuda(), cache)
    q8, w, _ = m.idx_quant_q_fold_w(torch.from_numpy(wl.q_bits(0).view(np.int16)).cuda(),
                                    torch.from_numpy(wl.w_raw(0)).cuda())
    nb, ns = wl.new_rows(0)
    k_new = torch.from_numpy(nb.view(np.int16)).cuda()
    slots = torch.from_numpy(ns).cuda()
    caches = [cache] + [m.KCache(wl.num_blocks, tensor=cache.tensor.clone()) for _ in range(replicas - 1)]
    torch.cuda.synchronize()
    log(f"setup {wl.name}: {time.time() - t0:.1f}s, {replicas} cache copies of "
        f"{cache.tensor.numel() / 1e6:.1f} MB")
    return dict(batch=batch, caches=caches, q8=q8, w=w, k_new=k_new, slots=slots)


def positions_sum(wl):
    return int(np.sum(wl.token_pos() + 1))


def algorithmic(wl):
    """Per-step algorithmic work: K bytes scored, HBM bytes of the step, MFMA flops."""
    P = positions_sum(wl)
    T = wl.num_tokens
    step_bytes = P * 132 + T * (64 * 128 + 64 * 4 + 4 * wl.k + 256 + 132)
    logits_bytes = P * (132 + 4) + T * (64 * 128 + 64 * 4)
    # each byte once: every request's K, q codes and weights in, one score out per position
    unique_bytes = int(np.sum(wl.seq_lens)) * 132 + T * (64 * 128 + 64 * 4) + P * 4
    flops = 2 * 64 * 128 * P
    return dict(positions=P, step_bytes=step_bytes, logits_bytes=logits_bytes,
                unique_bytes=unique_bytes, flops=flops)


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


def run_workload(m, torch, name, args):
    from synth import CONFIGS, make_workload
    wl = make_workload(CONFIGS[name])
    decode = wl.max_query_len == 1
    reps = args.replicas if decode else 1
    d = setup(m, torch, wl, reps)
    B, k = d["batch"], wl.k
    topk = torch.empty((wl.num_tokens, k), dtype=torch.int32, device="cuda")
    ws = torch.empty(m.idx_score_topk_workspace_size(B, k), dtype=torch.uint8, device="cuda")
    logits = torch.empty((wl.num_tokens, wl.max_seq_len), dtype=torch.float32, device="cuda")

    def step(i):                                       # one F layer: a1 + a4
        c = d["caches"][i % reps]
        m.idx_indexcache_layer(d["k_new"], c, d["q8"], d["w"], True, True, d["slots"], B, k, topk,
                               workspace=ws)

    def score_only(i):
        m.idx_logits(d["q8"], d["w"], d["caches"][i % reps], B, logits=logits)

    ms_step = time_loop(torch, step, args.steps, args.warmup)
    ms_logits = time_loop(torch, score_only, args.steps, args.warmup)
    a = algorithmic(wl)
    if decode:
        ach = a["logits_bytes"] / (ms_logits * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic("score_decode_kernel", name),
                "kernel": "score_decode_kernel (idx_logits)", "ms_per_launch": round(ms_logits, 5),
                "bytes_per_launch": a["logits_bytes"]}
    else:
        ach = a["flops"] / (ms_logits * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / FP8_PEAK_TFLOPS, 4),
                "traffic": measured_traffic("score_prefill_kernel", name),
                "kernel": "score_prefill_kernel (idx_logits)", "ms_per_launch": round(ms_logits, 5),
                "flops_per_launch": a["flops"]}
    step_gbs = a["step_bytes"] / (ms_step * 1e-3) / 1e9
    res = dict(workload=name, tokens=wl.num_tokens, ms_per_step=ms_step,
               value=wl.num_tokens / (ms_step * 1e-3), roofline=roof,
               step_hbm_frac=round(step_gbs / HBM_PEAK_GBS, 4),
               step_mfma_frac=round(a["flops"] / (ms_step * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 4),
               config={"workload": name, "requests": wl.num_reqs, "query_tokens": wl.num_tokens,
                       "max_context": wl.max_seq_len, "index_topk": k, "heads": 64, "head_dim": 128,
                       "block_size": 64, "cache_copies": reps})
    log(f"{name}: {ms_step * 1e3:.1f} us/step, logits kernel {ms_logits * 1e3:.1f} us "
        f"({roof['frac'] * 100:.1f}% of {roof['bound']} peak)")
    return res, wl


def cpu_baseline(wl, sample, min_seconds=10.0):
    """The oracle, as it stands, on `sample` query tokens of the workload, repeated
    until at least `min_seconds` of work has been timed."""
    import concurrent.futures as cf
    import oracle
    from oracle import logits as olog, quant as oquant, topk as otopk
    try:
        from threadpoolctl import threadpool_info
        blas = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        blas = None
    tokens = np.linspace(0, wl.num_tokens - 1, min(sample, wl.num_tokens)).astype(int)
    reqs = sorted(set(int(r) for r in wl.token_req()[tokens]))
    cache = np.zeros((wl.num_blocks, 64, 132), np.uint8)
    new = {}
    nw = max(1, min(16, len(os.sched_getaffinity(0))))
    with cf.ThreadPoolExecutor(nw) as ex:               # context: setup, not timed
        for r, kb in ex.map(lambda r: (r, wl.request_k(0, r)), reqs):
            L, n = int(wl.seq_lens[r]), int(wl.new_tokens[r])
            oquant.quant_write_k(cache, kb[:L - n], wl.slots(r, np.arange(L - n)))
            new[r] = (kb[L - n:], wl.slots(r, np.arange(L - n, L)))
    q8, qs = oquant.quantize_q(wl.q_bits(0))
    w = oquant.fold_weights(wl.w_raw(0), qs)
    ob = oracle.Batch(wl.seq_lens, wl.query_start_loc, wl.block_table)
    passes = 0
    t0 = time.time()
    while passes == 0 or time.time() - t0 < min_seconds:
        for r in reqs:                                 # this step's K rows of the sampled requests
            oquant.quant_write_k(cache, *new[r])
        for t in tokens:
            r, p = ob.token_request(int(t)), ob.token_position(int(t))
            s = olog.logits_row(q8[t], w[t], cache, wl.block_table[r], p)
            otopk.topk_row(s, wl.k)
        passes += 1
    dt = time.time() - t0
    return {"value": round(passes * len(tokens) / dt, 3), "unit": "query-tokens/s",
            "cores": len(os.sched_getaffinity(0)), "blas_threads": blas, "kind": "oracle",
            "sample": f"{passes} pass(es) over {len(tokens)} of the {wl.num_tokens} query tokens of "
                      f"{wl.name} (their new K rows, fp64 scores over the full causal range, "
                      f"full-sort top-{wl.k}); {dt:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); this build has no "
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
    main_res, wl = run_workload(m, torch, args.workload, args)
    out = {"metric": METRIC, "value": round(main_res["value"], 1), "unit": "query-tokens/s",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(main_res["ms_per_step"], 5), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "fp8e4m3", "data": "synthetic",
           "config": main_res["config"], "roofline": main_res["roofline"],
           "step_hbm_frac": main_res["step_hbm_frac"]}
    if args.secondary:
        sec, _ = run_workload(m, torch, args.secondary, args)
        out["secondary"] = {k: sec[k] for k in ("workload", "value", "ms_per_step", "roofline",
                                                 "step_mfma_frac", "config")}
        out["secondary"]["value"] = round(sec["value"], 1)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_sample, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
