"""Benchmark of the fused-attention hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--quick]

Headline (the JSON line's `value`): single-query GQA decode of the
Llama-3-8B-shaped workload (B=8, 32 query heads over 8 K/V heads, 4096 cached
tokens, d=128, bf16 cache, fp32 accumulation), in K/V-cache GB/s: the
algorithmic bytes of one call (K and V rows read once, q read, O and LSE
written) divided by the GPU time per call. A call is the library entry point
(split kernel + LSE merge kernel). Inputs are resident in HBM before the timed
region; consecutive steps rotate over several copies of the cache whose total
size exceeds twice the 256 MB Infinity Cache, so each step streams from HBM
rather than from the last-level cache. Steps are launched by replaying a HIP
graph of 20 consecutive calls, so host-side launch cost (Python and ctypes)
is not what is measured; the eager per-call time is reported beside it.

The same line also carries:
  * "roofline": the decode kernel's achieved bandwidth per launch (HIP events
    around every launch on the launch stream) against the 8 TB/s HBM peak,
    with the counter-measured HBM traffic when a matching counter summary is
    present under profiles/ (null otherwise);
  * "cpu_baseline": the fp64 oracle timed on this host's cores over repeated
    full passes of the same workload (a reported baseline, not a target);
  * "workloads": every named workload timed the same way, each priced against
    its roofline (prefill: unmasked-pair flops vs 2.5 PFLOP/s dense bf16 MFMA;
    decode: algorithmic bytes vs 8 TB/s HBM).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
FP32_VALU_PEAK_TFLOPS = 157.3
MALL_BYTES = 256 << 20
METRIC = "prefill TFLOP/s (% bf16 MFMA peak); decode KV GB/s (% of HBM peak)"
HEADLINE = "decode_gqa_llama3_8b_4k"
COUNTERS_FILE = os.path.join(ROOT, "profiles", "decode_gqa_llama3_8b_4k_counters.json")
DECODE_SRCS = [os.path.join(ROOT, "transformer_attention_05_amd", "csrc", f)
               for f in ("decode_gqa.hip", "merge.hip", "common.h")]


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quick", action="store_true", help="headline workload only")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--only", metavar="WORKLOAD",
                    help="time one named workload and print its result (for profiler runs)")
    ap.add_argument("--counters", action="store_true",
                    help="few headline launches + a calibration copy, for rocprofv3 --pmc runs")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                    help="write the counter summary of two --counters runs under profiles/")
    return ap.parse_args()


def _rotation(nbytes_per_set: int) -> int:
    """Copies needed so the rotation footprint exceeds twice the MALL."""
    return max(2, -(-2 * MALL_BYTES // max(1, nbytes_per_set)) + 1)


def _time_calls(torch, calls, steps, warmup, per_graph):
    """Time `steps` calls.

    After an eager warm-up, `per_graph` consecutive calls are captured into
    one HIP graph, which is replayed steps / per_graph times; the timed
    region is bracketed by synchronisation, and the GPU time comes from an
    event pair on the replay stream. The graph removes host launch overhead
    (Python + ctypes per call) from the measurement; every kernel of every
    call still runs. Also returns an eager per-call time for reference.
    Returns (wall seconds, GPU seconds, eager seconds per call).
    """
    n = len(calls)
    for i in range(warmup):
        calls[i % n]()
    torch.cuda.synchronize()
    ne = min(steps, 50)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(ne):
        calls[i % n]()
    e1.record()
    torch.cuda.synchronize()
    eager = e0.elapsed_time(e1) / 1e3 / ne
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(per_graph):
            calls[i % n]()
    g.replay()
    torch.cuda.synchronize()
    reps = steps // per_graph
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for _ in range(reps):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, start.elapsed_time(end) / 1e3, eager


def _upload_bf16(torch, bits, dev):
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def _upload_f32(torch, x, dev):
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev)


def bench_workload(torch, attn, workloads, name, steps, warmup, dev):
    """Time one named workload; returns a result dict."""
    cfg = workloads.WORKLOADS[name]
    w = workloads.make(name)
    kind = cfg["kind"]
    ragged = getattr(w, "kv_lens", None) is not None and kind != "prefill_chunked"
    if ragged:
        lens = torch.from_numpy(w.kv_lens).to(dev)
    if kind == "decode_gqa":
        fp8 = w.cache_dtype == "fp8"
        q = _upload_bf16(torch, w.q, dev)
        if fp8:
            k, v = (torch.from_numpy(x).to(dev) for x in (w.k, w.v))
        else:
            k, v = (_upload_bf16(torch, x, dev) for x in (w.k, w.v))
        if ragged:
            nbytes = workloads.decode_gqa_ragged_bytes(w.Hq, w.Hkv, w.kv_lens, w.D)
        else:
            nbytes = workloads.decode_gqa_bytes(w.B, w.Hq, w.Hkv, w.kv_len, w.D,
                                                kv_elt=1 if fp8 else 2)
        sets = [(q, k, v)] + [(q, k.clone(), v.clone())
                              for _ in range(_rotation(2 * k.numel() * k.element_size()) - 1)]
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device=dev)
        ws = torch.empty(attn.attn_decode_gqa_workspace_bytes(w.B, w.Hq, w.Hkv, w.kv_len, w.D),
                         dtype=torch.uint8, device=dev)
        if ragged:
            calls = [lambda s=s: attn.attn_decode_gqa_ragged(s[0], s[1], s[2], lens, w.kv_len,
                                                             w.scale, out=o, lse=lse, ws=ws)
                     for s in sets]
        elif fp8:
            calls = [lambda s=s: attn.attn_decode_gqa_fp8(s[0], s[1], s[2], w.kv_len, w.scale, out=o,
                                                          lse=lse, ws=ws) for s in sets]
        else:
            calls = [lambda s=s: attn.attn_decode_gqa(s[0], s[1], s[2], w.kv_len, w.scale, out=o,
                                                      lse=lse, ws=ws) for s in sets]
        work, unit, peak, bound = nbytes / 1e9, "GB/s", HBM_PEAK_GBS, "hbm"
        kernel = "decode_gqa_kernel<%s> + merge_kernel" % ("true" if fp8 else "false")
    elif kind == "decode_mla":
        fp8 = w.cache_dtype == "fp8"
        q = _upload_bf16(torch, w.q, dev)
        c = torch.from_numpy(w.ckv).to(dev) if fp8 else _upload_bf16(torch, w.ckv, dev)
        if ragged:
            nbytes = workloads.decode_mla_ragged_bytes(w.Hq, w.kv_lens, w.Dqk, w.Dv)
        else:
            nbytes = workloads.decode_mla_bytes(w.B, w.Hq, w.kv_len, w.Dqk, w.Dv,
                                                kv_elt=1 if fp8 else 2)
        sets = [(q, c)] + [(q, c.clone())
                           for _ in range(_rotation(c.numel() * c.element_size()) - 1)]
        o = torch.empty((w.B, w.Hq, w.Dv), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device=dev)
        ws_fn = attn.attn_decode_mla_ragged_workspace_bytes if ragged else attn.attn_decode_mla_workspace_bytes
        ws = torch.empty(ws_fn(w.B, w.Hq, w.kv_len, w.Dqk, w.Dv), dtype=torch.uint8, device=dev)
        if ragged:
            calls = [lambda s=s: attn.attn_decode_mla_ragged(s[0], s[1], lens, w.kv_len, w.Dv,
                                                             w.scale, out=o, lse=lse, ws=ws)
                     for s in sets]
        elif fp8:
            calls = [lambda s=s: attn.attn_decode_mla_fp8(s[0], s[1], w.kv_len, w.Dv, w.scale,
                                                          out=o, lse=lse, ws=ws) for s in sets]
        else:
            calls = [lambda s=s: attn.attn_decode_mla_absorbed(s[0], s[1], w.kv_len, w.Dv, w.scale,
                                                               out=o, lse=lse, ws=ws) for s in sets]
        work, unit, peak, bound = nbytes / 1e9, "GB/s", HBM_PEAK_GBS, "hbm"
        kernel = "decode_mla_kernel%s + merge_kernel" % ("<E4M3>" if fp8 else "")
    elif kind == "prefill_backward":
        q, k, v = (_upload_bf16(torch, x, dev) for x in (w.q, w.k, w.v))
        dout = _upload_bf16(torch, workloads.gen_upstream_grad((w.B, w.Hq, w.N, w.D), seed=1010), dev)
        o, lse = attn.attn_prefill_causal(q, k, v, w.scale)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(attn.attn_prefill_causal_backward_workspace_bytes(w.B, w.Hq, w.N, w.D),
                         dtype=torch.uint8, device=dev)
        flops = workloads.prefill_backward_flops(w.B, w.Hq, w.N, w.D)
        calls = [lambda: attn.attn_prefill_causal_backward(q, k, v, o, lse, dout, w.scale, dq=dq,
                                                           dk=dk, dv=dv, ws=ws)]
        work, unit, peak, bound = flops / 1e12, "TFLOP/s", MFMA_BF16_PEAK_TFLOPS, "mfma"
        kernel = "bwd_dot_kernel + bwd_dkdv_kernel + bwd_dq_kernel"
        nsteps = max(5, min(steps, int(1e14 // max(flops, 1))))
        if nsteps >= 20:
            nsteps -= nsteps % 20
        steps, warmup = nsteps, max(min(warmup, 5), min(200, int(2e13 // max(flops, 1))))
    elif kind == "prefill_chunked":
        q, k, v = (_upload_bf16(torch, x, dev) for x in (w.q, w.k, w.v))
        lens = torch.from_numpy(w.kv_lens).to(dev)
        flops = workloads.prefill_chunked_flops(w.Hq, w.Nq, w.kv_lens, w.D)
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device=dev)
        ws = torch.empty(attn.attn_prefill_chunked_workspace_bytes(w.B, w.Hq, w.Nq, w.kv_cap, w.D),
                         dtype=torch.uint8, device=dev)
        calls = [lambda: attn.attn_prefill_chunked(q, k, v, lens, w.scale, out=o, lse=lse, ws=ws)]
        work, unit, peak, bound = flops / 1e12, "TFLOP/s", MFMA_BF16_PEAK_TFLOPS, "mfma"
        kernel = "prefill_d128_kernel<true>" + (
            " + merge_kernel" if attn.attn_prefill_chunked_workspace_bytes(
                w.B, w.Hq, w.Nq, w.kv_cap, w.D) > 256 else "")
        nsteps = max(5, min(steps, int(1e14 // max(flops, 1))))
        if nsteps >= 20:
            nsteps -= nsteps % 20
        steps, warmup = nsteps, max(min(warmup, 5), min(200, int(2e13 // max(flops, 1))))
    else:
        up = _upload_bf16 if w.dtype == "bf16" else _upload_f32
        q, k, v = (up(torch, x, dev) for x in (w.q, w.k, w.v))
        flops = workloads.prefill_causal_flops(w.B, w.Hq, w.N, w.D)
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=dev)
        calls = [lambda: attn.attn_prefill_causal(q, k, v, w.scale, out=o, lse=lse)]
        work = flops / 1e12
        unit = "TFLOP/s"
        if w.dtype == "bf16":
            peak, bound = MFMA_BF16_PEAK_TFLOPS, "mfma"
            kernel = "prefill_d128_kernel<false>" if w.D == 128 else "prefill_bf16_kernel"
        else:
            peak, bound, kernel = FP32_VALU_PEAK_TFLOPS, "alu", "prefill_f32_kernel"
        # about 0.1 s of timed work after about 20 ms of warm-up (the clocks
        # ramp during the first milliseconds of a burst)
        nsteps = max(5, min(steps, int(1e14 // max(flops, 1))))
        if nsteps >= 20:
            nsteps -= nsteps % 20
        steps, warmup = nsteps, max(min(warmup, 5), min(200, int(2e13 // max(flops, 1))))
    per_graph = 20 if steps % 20 == 0 else 1
    wall, gpu, eager = _time_calls(torch, calls, steps, warmup, per_graph)
    per = gpu / steps
    return dict(kernel=kernel, steps=steps, calls_per_graph=per_graph,
                ms_per_call=1e3 * per, wall_ms_per_call=1e3 * wall / steps,
                eager_ms_per_call=1e3 * eager, value=work / per, unit=unit, bound=bound,
                achieved=work / per, peak=peak, frac=work / per / peak,
                work_per_call=(nbytes if unit == "GB/s" else flops))


def _decode_source_hash() -> str:
    h = hashlib.sha256()
    for f in DECODE_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def _traffic():
    """HBM bytes per call from the committed counter summary, if it was taken
    on the current decode kernel sources (else None)."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    try:
        rec = json.load(open(COUNTERS_FILE))
        if rec.get("source_sha256") != _decode_source_hash():
            return None
        return rec.get("hbm_bytes_per_call")
    except (OSError, ValueError):
        return None


def summarize_counters(fetch_db: str, write_db: str) -> dict:
    """Turn the two `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs of
    `bench.py --counters` into HBM bytes per decode call.

    Each counter (KiB per dispatch) is scaled by the factor that makes it read
    CALIB_BYTES for the calibration copy (the last copy dispatch of the run).
    The decode call's kernels are the split kernel and the merge kernel."""
    import sqlite3

    def per_kernel(db, counter):
        rows = sqlite3.connect(db).execute(
            "select kernel_name, value from counters_collection where counter_name = ? "
            "order by dispatch_id", (counter,)).fetchall()
        copies = [v for n, v in rows if "copyBuffer" in n]
        scale = CALIB_BYTES / (copies[-1] * 1024.0)
        out = {}
        for n, v in rows:
            for key in ("decode_gqa_kernel", "merge_kernel"):
                if key in n:
                    out.setdefault(key, []).append(v * 1024.0 * scale)
        return scale, {k: sum(v) / len(v) for k, v in out.items()}, {k: len(v) for k, v in out.items()}

    fs, fetch, nf = per_kernel(fetch_db, "FETCH_SIZE")
    ws, write, nw = per_kernel(write_db, "WRITE_SIZE")
    total = sum(fetch.values()) + sum(write.values())
    return {
        "workload": HEADLINE, "source_sha256": _decode_source_hash(),
        "fetch_scale": round(fs, 5), "write_scale": round(ws, 5),
        "fetch_bytes": {k: round(v) for k, v in fetch.items()},
        "write_bytes": {k: round(v) for k, v in write.items()},
        "dispatches": {"fetch": nf, "write": nw},
        "hbm_bytes_per_call": round(total),
        "algorithmic_bytes_per_call": 134349824,
        "commands": ["rocprofv3 --pmc FETCH_SIZE -d prof/fetch -o fetch -- python3 -u bench.py --counters",
                     "rocprofv3 --pmc WRITE_SIZE -d prof/write -o write -- python3 -u bench.py --counters",
                     "python3 bench.py --summarize-counters prof/fetch/fetch_results.db "
                     "prof/write/write_results.db"],
    }


def cpu_baseline(workloads, seconds):
    """The fp64 oracle on this host over repeated full passes of the headline
    workload; GB/s of the same algorithmic bytes."""
    import oracle
    w = workloads.make(HEADLINE)
    nbytes = workloads.decode_gqa_bytes(w.B, w.Hq, w.Hkv, w.kv_len, w.D)
    threads = oracle.default_threads()
    oracle.decode_gqa(w.q[:1, :, :], w.k[:1, :, :64], w.v[:1, :, :64], 64, w.scale, threads=threads)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.decode_gqa(w.q, w.k, w.v, w.kv_len, w.scale, threads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return dict(value=reps * nbytes / el / 1e9, unit="GB/s", cores=threads, kind="oracle",
                sample="%d full passes of %s (B=8, Hq=32, Hkv=8, kv_len=4096, d=128) in %.1f s, "
                       "fp64, bf16 inputs widened per pass" % (reps, HEADLINE, el))


CALIB_BYTES = 512 << 20


def counters_run(torch, attn, workloads, dev):
    """Launch the headline decode kernel 5 times (one input set per launch,
    so every launch streams from HBM) and one plain copy of CALIB_BYTES, whose
    FETCH_SIZE / WRITE_SIZE calibrate the counters against a known size."""
    w = workloads.make(HEADLINE)
    q = _upload_bf16(torch, w.q, dev)
    k0, v0 = _upload_bf16(torch, w.k, dev), _upload_bf16(torch, w.v, dev)
    sets = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(4)]
    torch.cuda.synchronize()
    for k, v in sets:
        attn.attn_decode_gqa(q, k, v, w.kv_len, w.scale)
        torch.cuda.synchronize()
        print("decode launch done", flush=True)
    src = torch.empty(CALIB_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    scrub = torch.empty((1 << 30) // 4, dtype=torch.float32, device=dev).fill_(2.0)  # evict src
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del scrub
    print("calibration copy of %d bytes done" % CALIB_BYTES, flush=True)


def main():
    a = _args()
    if a.summarize_counters:
        rec = summarize_counters(*a.summarize_counters)
        with open(COUNTERS_FILE, "w") as f:
            json.dump(rec, f, indent=1)
        print(json.dumps(rec))
        return
    if a.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % a.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    import transformer_attention_05_amd as attn
    import workloads
    attn.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if a.counters:
        counters_run(torch, attn, workloads, dev)
        return
    if a.only:
        r = bench_workload(torch, attn, workloads, a.only, a.steps, a.warmup, dev)
        print(json.dumps({a.only: r}), flush=True)
        return

    head = bench_workload(torch, attn, workloads, HEADLINE, a.steps, a.warmup, dev)
    print("headline %s: %.1f GB/s, %.4f ms per call (eager launches: %.4f ms)" % (
        HEADLINE, head["value"], head["ms_per_call"], head["eager_ms_per_call"]),
        file=sys.stderr, flush=True)
    results = {HEADLINE: head}
    if not a.quick:
        for name in workloads.WORKLOADS:
            if name == HEADLINE:
                continue
            torch.cuda.empty_cache()
            r = bench_workload(torch, attn, workloads, name, a.steps, a.warmup, dev)
            results[name] = r
            print("%s: %.2f %s (%.1f %% of %s peak), %.3f ms" % (
                name, r["value"], r["unit"], 100 * r["frac"], r["bound"], r["ms_per_call"]),
                file=sys.stderr, flush=True)

    cpu = None if a.no_cpu_baseline else cpu_baseline(workloads, a.cpu_seconds)
    w = workloads.WORKLOADS[HEADLINE]
    line = {
        "metric": METRIC, "value": round(head["value"], 2), "unit": "GB/s", "n_gpus": 1,
        "steps": head["steps"], "warmup": a.warmup, "ms_per_step": round(head["ms_per_call"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": HEADLINE, "B": w["B"], "Hq": w["Hq"], "Hkv": w["Hkv"],
                   "kv_len": w["kv_len"], "D": w["D"], "cache_dtype": "bf16",
                   "accumulate": "fp32", "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "kernel": head["kernel"],
                     "achieved": round(head["achieved"], 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(head["frac"], 4), "traffic": _traffic(),
                     "bytes_per_launch": head["work_per_call"]},
        "cpu_baseline": None if cpu is None else {k: (round(v, 4) if isinstance(v, float) else v)
                                                  for k, v in cpu.items()},
        "workloads": {n: {k: (round(v, 5) if isinstance(v, float) else v) for k, v in r.items()}
                      for n, r in results.items()},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
