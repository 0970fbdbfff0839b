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
    decode: algorithmic bytes vs 8 TB/s HBM), each with its own cpu_baseline
    (the oracle on a bounded sample of that workload, the sample and any
    extrapolation stated; the tiny prefill and the Llama-3 decode also on one
    core) and, where a counter summary for the current sources exists under
    profiles/, the HBM traffic per call;
  * "ceilings": what this GPU does on a plain streaming read (the read
    bandwidth a decode can hope for) and the issue cost of v_exp_f32, of an
    fp32 FMA and of a 2^x built from FMAs (libattn_probes.so).

Other modes: --only NAME (one workload), --ceilings (the probes alone),
--counters [--only NAME] (a few launches and a calibration copy, for
rocprofv3 --pmc runs), --summarize-counters FETCH_DB WRITE_DB [--only NAME].
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
                    help="few launches of the headline (or --only) workload + a calibration copy, "
                         "for rocprofv3 --pmc runs")
    ap.add_argument("--ceilings", action="store_true",
                    help="run the streaming-read and VALU-issue probes and print their results")
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


def bench_workload(torch, attn, workloads, name, steps, warmup, dev, plain=False, w=None):
    """Time one named workload; returns a result dict. plain: launch `steps`
    calls eagerly and time them, nothing more (for counter runs). w: the
    workload's inputs, if already made."""
    cfg = workloads.WORKLOADS[name]
    w = workloads.make(name) if w is None else w
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
            nbytes = workloads.decode_mla_ragged_bytes(w.Hq, w.kv_lens, w.Dqk, w.Dv,
                                                       kv_elt=1 if fp8 else 2)
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
            fn = attn.attn_decode_mla_ragged_fp8 if fp8 else attn.attn_decode_mla_ragged
            calls = [lambda s=s: fn(s[0], s[1], lens, w.kv_len, w.Dv, w.scale, out=o, lse=lse,
                                    ws=ws)
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
    if plain:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            calls[i % len(calls)]()
            torch.cuda.synchronize()
        return dict(ms_per_call=1e3 * (time.perf_counter() - t0) / steps)
    per_graph = 20 if steps % 20 == 0 else 1
    wall, gpu, eager = _time_calls(torch, calls, steps, warmup, per_graph)
    per = gpu / steps
    return dict(kernel=kernel, steps=steps, calls_per_graph=per_graph,
                ms_per_call=1e3 * per, wall_ms_per_call=1e3 * wall / steps,
                eager_ms_per_call=1e3 * eager, value=work / per, unit=unit, bound=bound,
                achieved=work / per, peak=peak, frac=work / per / peak,
                work_per_call=(nbytes if unit == "GB/s" else flops))


# sources of each workload kind's kernels (paths under csrc/): a counter
# summary counts only while they are unchanged. The GQA decode also names
# build.py, which gives its bf16 unit a compile option of its own.
KIND_SRCS = {
    "decode_gqa": ("decode_gqa_kernel.h", "decode_gqa.hip", "decode_gqa_fp8.hip", "merge.hip",
                   "common.h", "ragged.h", "../build.py"),
    "decode_mla": ("decode_mla.hip", "merge.hip", "common.h", "ragged.h"),
    "prefill": ("prefill_bf16_d128.hip", "prefill_bf16.hip", "prefill_f32.hip", "common.h"),
    "prefill_chunked": ("prefill_bf16_d128.hip", "merge.hip", "common.h"),
    "prefill_backward": ("prefill_bwd_d128.hip", "common.h"),
}
# kernel-name pieces of each kind's launches
KIND_KERNELS = {
    "decode_gqa": ("decode_gqa_kernel", "merge_kernel", "merge_ragged_kernel"),
    "decode_mla": ("decode_mla_kernel", "merge_kernel", "merge_ragged_kernel"),
    "prefill": ("prefill_d128_kernel", "prefill_bf16_kernel", "prefill_f32_kernel"),
    "prefill_chunked": ("prefill_d128_kernel", "merge_kernel"),
    "prefill_backward": ("bwd_dot_kernel", "bwd_dkdv_kernel", "bwd_dq_kernel"),
}


def _counters_file(name):
    return os.path.join(ROOT, "profiles", "%s_counters.json" % name)


def _source_hash(kind) -> str:
    h = hashlib.sha256()
    for f in KIND_SRCS[kind]:
        h.update(open(os.path.join(ROOT, "transformer_attention_05_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def _traffic(name, kind):
    """HBM bytes per call from the committed counter summary of this
    workload, if it was taken on the current kernel sources (else None)."""
    path = _counters_file(name)
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
        if rec.get("source_sha256") != _source_hash(kind):
            return None
        return rec.get("hbm_bytes_per_call")
    except (OSError, ValueError):
        return None


def summarize_counters(fetch_db: str, write_db: str, name: str) -> dict:
    """Turn the two `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs of
    `bench.py --counters --only NAME` into HBM bytes per call.

    Each counter (KiB per dispatch) is scaled by the factor that makes it read
    CALIB_BYTES for the calibration copy (the last copy dispatch of the run).
    A call is every kernel of the workload's kind, averaged per dispatch."""
    import sqlite3
    import workloads
    kind = workloads.WORKLOADS[name]["kind"]

    def per_kernel(db, counter):
        rows = sqlite3.connect(db).execute(
            "select kernel_name, value from counters_collection where counter_name = ? "
            "order by dispatch_id", (counter,)).fetchall()
        copies = [v for n, v in rows if "copyBuffer" in n]
        scale = CALIB_BYTES / (copies[-1] * 1024.0)
        out = {}
        for n, v in rows:
            for key in KIND_KERNELS[kind]:
                if key in n and "copyBuffer" not in n:
                    out.setdefault(key, []).append(v * 1024.0 * scale)
                    break
        return scale, {k: sum(v) / len(v) for k, v in out.items()}, {k: len(v) for k, v in out.items()}

    fs, fetch, nf = per_kernel(fetch_db, "FETCH_SIZE")
    ws, write, nw = per_kernel(write_db, "WRITE_SIZE")
    total = sum(fetch.values()) + sum(write.values())
    w = workloads.make(name)
    algo = _work_bytes(workloads, name, w)
    return {
        "workload": name, "source_sha256": _source_hash(kind),
        "fetch_scale": round(fs, 5), "write_scale": round(ws, 5),
        "fetch_bytes": {k: round(v) for k, v in fetch.items()},
        "write_bytes": {k: round(v) for k, v in write.items()},
        "dispatches": {"fetch": nf, "write": nw},
        "hbm_bytes_per_call": round(total),
        "algorithmic_bytes_per_call": algo,
        "traffic_over_algorithmic": None if not algo else round(total / algo, 4),
        "commands": ["rocprofv3 --pmc FETCH_SIZE -d prof/ctr/%s/fetch -o fetch -- python3 -u "
                     "bench.py --counters --only %s" % (name, name),
                     "rocprofv3 --pmc WRITE_SIZE -d prof/ctr/%s/write -o write -- python3 -u "
                     "bench.py --counters --only %s" % (name, name),
                     "python3 bench.py --summarize-counters prof/ctr/%s/fetch/fetch_results.db "
                     "prof/ctr/%s/write/write_results.db --only %s" % (name, name, name)],
    }


def _work_bytes(workloads, name, w):
    """Algorithmic HBM bytes of one call of a decode workload (None otherwise)."""
    kind = workloads.WORKLOADS[name]["kind"]
    ragged = getattr(w, "kv_lens", None) is not None and kind != "prefill_chunked"
    if kind == "decode_gqa":
        if ragged:
            return workloads.decode_gqa_ragged_bytes(w.Hq, w.Hkv, w.kv_lens, w.D)
        return workloads.decode_gqa_bytes(w.B, w.Hq, w.Hkv, w.kv_len, w.D,
                                          kv_elt=1 if w.cache_dtype == "fp8" else 2)
    if kind == "decode_mla":
        if ragged:
            return workloads.decode_mla_ragged_bytes(w.Hq, w.kv_lens, w.Dqk, w.Dv,
                                                     kv_elt=1 if w.cache_dtype == "fp8" else 2)
        return workloads.decode_mla_bytes(w.B, w.Hq, w.kv_len, w.Dqk, w.Dv,
                                          kv_elt=1 if w.cache_dtype == "fp8" else 2)
    return None


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


def _timed(fn, seconds):
    """Run fn() repeatedly for about `seconds` (at least once); return the
    number of runs and the elapsed time."""
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            return reps, el


def cpu_baseline_for(workloads, name, w, seconds, threads):
    """The fp64 oracle on a bounded sample of workload `name` (input w), in
    the workload's own unit. Decodes with a small cache run whole; long
    prefills run a stratified set of query rows (the first, the last, and
    evenly spaced ones), MLA decodes a subset of the heads of one sequence,
    the backward a causal prefix of one (b, K/V head) group; each sample's
    time is scaled up to the whole workload by its share of the work (visible
    (query, key) pairs, or heads), and that is said in `sample`."""
    import numpy as np
    import oracle
    cfg = workloads.WORKLOADS[name]
    kind = cfg["kind"]
    ragged = getattr(w, "kv_lens", None) is not None and kind != "prefill_chunked"
    rec = dict(cores=threads, kind="oracle")
    if kind == "decode_gqa":
        nbytes = _work_bytes(workloads, name, w)
        if ragged:
            fn = lambda: oracle.decode_gqa_ragged(w.q, w.k, w.v, w.kv_lens, w.scale, threads=threads)
        else:
            fn = lambda: oracle.decode_gqa(w.q, w.k, w.v, w.kv_len, w.scale, threads=threads)
        reps, el = _timed(fn, seconds)
        rec.update(value=reps * nbytes / el / 1e9, unit="GB/s", extrapolated=False,
                   sample="%d full passes in %.1f s" % (reps, el))
        return rec
    if kind == "decode_mla":
        nbytes = _work_bytes(workloads, name, w)
        heads = 16
        b = int(np.argmax(w.kv_lens)) if ragged else 0
        L = int(w.kv_lens[b]) if ragged else w.kv_len
        q1, c1 = w.q[b:b + 1, :heads], w.ckv[b:b + 1]
        fn = lambda: oracle.decode_mla_absorbed(q1, c1, L, w.Dv, w.scale, threads=threads)
        reps, el = _timed(fn, seconds)
        # share of the work: heads × keys of the sample over all (b, head, key)
        keys_all = int(np.sum(w.kv_lens)) if ragged else w.B * w.kv_len
        share = heads * L / (w.Hq * keys_all)
        t_full = el / reps / share
        rec.update(value=nbytes / t_full / 1e9, unit="GB/s", extrapolated=True,
                   full_seconds=round(t_full, 2),
                   sample="%d heads of sequence %d (%d keys), %d passes in %.1f s, scaled by "
                          "heads x keys to the whole batch" % (heads, b, L, reps, el))
        return rec
    if kind == "prefill_backward":
        Np = min(w.N, 1024)
        G = w.Hq // w.Hkv
        dout = workloads.gen_upstream_grad((1, G, Np, w.D), seed=1010)
        qs, ks, vs = w.q[:1, :G, :Np], w.k[:1, :1, :Np], w.v[:1, :1, :Np]
        fn = lambda: oracle.prefill_causal_backward_rows(qs, ks, vs, dout, w.scale, threads=threads)
        reps, el = _timed(fn, seconds)
        flops_s = workloads.prefill_backward_flops(1, G, Np, w.D)
        flops = workloads.prefill_backward_flops(w.B, w.Hq, w.N, w.D)
        t_full = el / reps * flops / flops_s
        rec.update(value=flops / t_full / 1e12, unit="TFLOP/s", extrapolated=True,
                   full_seconds=round(t_full, 1),
                   sample="the first %d positions of one (b, K/V head) group (%d query heads), %d "
                          "passes in %.1f s, scaled by visible pairs" % (Np, G, reps, el))
        return rec
    # prefills: all rows when small, else a stratified row sample
    if kind == "prefill_chunked":
        Nq = w.Nq
        past = int(w.kv_lens[0]) - Nq
        flops = workloads.prefill_chunked_flops(w.Hq, w.Nq, w.kv_lens, w.D)
        pairs_of = lambda rows: np.sum(past + np.asarray(rows) + 1)
        run = lambda rows: oracle.prefill_chunked(w.q, w.k, w.v, w.kv_lens, w.scale, rows=rows,
                                                  threads=threads)
    else:
        Nq = w.N
        flops = workloads.prefill_causal_flops(w.B, w.Hq, w.N, w.D)
        pairs_of = lambda rows: np.sum(np.asarray(rows) + 1)
        run = lambda rows: oracle.prefill_causal(w.q, w.k, w.v, w.scale, rows=rows, threads=threads)
    total_pairs = (Nq * (Nq + 1) // 2 + (Nq * past if kind == "prefill_chunked" else 0)) * w.B * w.Hq
    if flops <= 2e9:  # small enough to run whole (about a second on a few cores)
        rows = np.arange(Nq, dtype=np.int32)
    else:
        rows = np.unique(np.concatenate([[0, Nq - 1], np.linspace(0, Nq - 1, 62).astype(np.int32)]))
    reps, el = _timed(lambda: run(rows), seconds)
    share = pairs_of(rows) * w.B * w.Hq / total_pairs
    t_full = el / reps / share
    whole = len(rows) == Nq
    rec.update(value=flops / t_full / 1e12, unit="TFLOP/s", extrapolated=not whole,
               full_seconds=round(t_full, 2),
               sample=("%d full passes in %.1f s" % (reps, el)) if whole else
                      ("%d query rows of %d (the first, the last, evenly spaced), every head, %d "
                       "passes in %.1f s, scaled by visible pairs" % (len(rows), Nq, reps, el)))
    return rec


def ceilings(torch, dev):
    """The probes of libattn_probes.so: best streaming-read rate over a few
    grid sizes at two buffer sizes, and the issue cost (shader-clock cycles per
    wave instruction per SIMD, 16 waves per CU) of v_exp_f32, an fp32 FMA and a
    2^x made of FMAs."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "transformer_attention_05_amd", "libattn_probes.so"))
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.attn_probe_stream_read.argtypes = [vp, sz, i, vp, vp]
    lib.attn_probe_valu.argtypes = [i, i, i, vp, vp, vp]
    lib.attn_probe_stream_ranges.argtypes = [vp, sz, i, i, i, vp, vp]
    lib.attn_probe_mfma_valu.argtypes = [i, i, i, i, vp, vp, vp]
    lib.attn_probe_lds_read.argtypes = [i, i, i, i, vp, vp, vp]
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    out = {}
    for mib in (128, 512):
        nbytes = mib << 20
        bufs = [torch.empty(nbytes // 4, dtype=torch.int32, device=dev).fill_(k) for k in range(3)]
        best = (0.0, 0)
        for blocks in (256, 512, 1024, 2048, 4096):
            for k in range(3):
                lib.attn_probe_stream_read(vp(bufs[k].data_ptr()), nbytes, blocks, vp(sink.data_ptr()), st)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = 12
            e0.record()
            for r in range(reps):
                lib.attn_probe_stream_read(vp(bufs[r % 3].data_ptr()), nbytes, blocks, vp(sink.data_ptr()), st)
            e1.record()
            torch.cuda.synchronize()
            gbs = nbytes * reps / (e0.elapsed_time(e1) / 1e3) / 1e9
            best = max(best, (gbs, blocks))
        out["stream_read_%dMiB_GBs" % mib] = round(best[0], 1)
        out["stream_read_%dMiB_blocks" % mib] = best[1]
        if mib == 128:
            # each workgroup streams its own range, as a decode split does:
            # µs per 128 MiB by workgroups x threads x loads per batch per lane
            ranges = {}
            for blocks, threads, inflight in ((64, 256, 32), (64, 1024, 8), (128, 256, 32),
                                              (128, 1024, 8), (256, 256, 8), (256, 256, 16),
                                              (256, 256, 32)):
                def go(k):
                    rc = lib.attn_probe_stream_ranges(vp(bufs[k % 3].data_ptr()), nbytes, blocks,
                                                      threads, inflight, vp(sink.data_ptr()), st)
                    assert rc == 0, rc
                for k in range(3):
                    go(k)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                reps = 12
                e0.record()
                for r in range(reps):
                    go(r)
                e1.record()
                torch.cuda.synchronize()
                ranges["%dx%dx%d" % (blocks, threads, inflight)] = round(e0.elapsed_time(e1) * 1e3 / reps, 1)
            out["stream_ranges_128MiB_us"] = ranges
        del bufs
    blocks, iters = 1024, 4096
    res = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    cyc = torch.zeros(blocks * 4, dtype=torch.int64, device=dev)
    for kind, key in ((0, "v_exp_f32"), (1, "fma_f32"), (2, "exp2_from_fma")):
        for r in range(2):
            lib.attn_probe_valu(kind, blocks, iters, vp(res.data_ptr()), vp(cyc.data_ptr()), st)
        torch.cuda.synchronize()
        per_wave = cyc.double().mean().item()
        waves_per_simd = blocks * 4 / 1024.0  # 256 CUs x 4 SIMDs
        out["cycles_per_wave_op_%s" % key] = round(per_wave / (iters * 8) / waves_per_simd, 2)
    # one wave per SIMD: shader-clock cycles per step of MFMAs (32x32x16 bf16)
    # plus independent fp32 FMAs
    blocks, iters = 1024, 2000
    res = torch.empty(blocks * 64, dtype=torch.float32, device=dev)
    cyc = torch.zeros(blocks, dtype=torch.int64, device=dev)
    steps = {}
    for mf, nv in ((1, 0), (1, 4), (1, 8), (1, 16), (2, 8), (2, 16), (0, 8), (0, 16)):
        for r in range(2):
            rc = lib.attn_probe_mfma_valu(mf, nv, blocks, iters, vp(res.data_ptr()), vp(cyc.data_ptr()), st)
            assert rc == 0, rc
        torch.cuda.synchronize()
        steps["%d_mfma_%d_fma" % (mf, nv)] = round(cyc.double().median().item() / (iters * 4), 1)
    out["cycles_per_step_one_wave"] = steps
    # LDS read rate per CU, one workgroup of 8 or 16 waves per CU
    blocks, iters = 256, 4096
    lds = {}
    for kind, key, nbytes in ((0, "ds_read_b128", 16), (1, "ds_read_b64_tr_b16", 8)):
        for threads in (512, 1024):
            res = torch.empty(blocks * threads, dtype=torch.int32, device=dev)
            cyc = torch.zeros(blocks * threads // 64, dtype=torch.int64, device=dev)
            for r in range(2):
                rc = lib.attn_probe_lds_read(kind, threads, blocks, iters, vp(res.data_ptr()),
                                             vp(cyc.data_ptr()), st)
                assert rc == 0, rc
            torch.cuda.synchronize()
            waves = threads // 64
            # a workgroup's waves start together after its fill; its slowest
            # wave spans the CU's reads
            span = cyc.double().view(blocks, waves).max(dim=1).values.median().item()
            lds["%s_%dwaves" % (key, waves)] = round(waves * iters * 8 * 64 * nbytes / span, 1)
    out["lds_read_bytes_per_clock_per_cu"] = lds
    out["note"] = ("stream read: best over 256..4096 workgroups, 16-byte non-temporal loads, "
                   "rotating three buffers; stream ranges: workgroups x threads x 16-byte loads "
                   "per lane issued as one batch, each workgroup reading its own contiguous range; "
                   "cycles: 16 waves per CU, eight independent chains per "
                   "lane, per 2^x (or FMA) per SIMD; one-wave steps: MFMAs into four "
                   "accumulators and FMAs in eight chains, median over 1024 waves; LDS reads: "
                   "eight per wave in flight, conflict-free addresses, bytes of all the CU's waves "
                   "over its slowest wave's cycles, median over CUs")
    return out


CALIB_BYTES = 512 << 20


def counters_run(torch, attn, workloads, dev, name):
    """Launch workload `name` 5 times (for a decode, one input set per launch so
    every launch streams from HBM) and one plain copy of CALIB_BYTES, whose
    FETCH_SIZE / WRITE_SIZE calibrate the counters against a known size."""
    r = bench_workload(torch, attn, workloads, name, 5, 1, dev, plain=True)
    print("%s: 5 launches done (%.3f ms per call)" % (name, r["ms_per_call"]), flush=True)
    src = torch.empty(CALIB_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    scrub = torch.empty((1 << 30) // 4, dtype=torch.float32, device=dev).fill_(2.0)  # evict src
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del scrub
    print("calibration copy of %d bytes done" % CALIB_BYTES, flush=True)


def _rounded(r):
    return {k: (round(v, 5) if isinstance(v, float) else
                (_rounded(v) if isinstance(v, dict) else v)) for k, v in r.items()}


def main():
    a = _args()
    if a.summarize_counters:
        name = a.only or HEADLINE
        rec = summarize_counters(*a.summarize_counters, name)
        with open(_counters_file(name), "w") as f:
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
        counters_run(torch, attn, workloads, dev, a.only or HEADLINE)
        return
    if a.ceilings:
        print(json.dumps(ceilings(torch, dev)), flush=True)
        return
    if a.only:
        r = bench_workload(torch, attn, workloads, a.only, a.steps, a.warmup, dev)
        print(json.dumps({a.only: r}), flush=True)
        return

    import oracle
    threads = oracle.default_threads()
    names = [HEADLINE] + ([] if a.quick else [n for n in workloads.WORKLOADS if n != HEADLINE])
    results = {}
    for name in names:
        torch.cuda.empty_cache()
        w = workloads.make(name)
        r = bench_workload(torch, attn, workloads, name, a.steps, a.warmup, dev, w=w)
        kind = workloads.WORKLOADS[name]["kind"]
        r["traffic"] = _traffic(name, kind)
        print("%s: %.2f %s (%.1f %% of %s peak), %.4f ms per call" % (
            name, r["value"], r["unit"], 100 * r["frac"], r["bound"], r["ms_per_call"]),
            file=sys.stderr, flush=True)
        if not a.no_cpu_baseline:
            # the oracle on a bounded sample: a couple of seconds per workload
            r["cpu_baseline"] = cpu_baseline_for(workloads, name, w, 2.0, threads)
            if name in (HEADLINE, "prefill_f32_tiny"):
                r["cpu_baseline_1core"] = cpu_baseline_for(workloads, name, w, 2.0, 1)
            print("  oracle: %.4g %s on %d cores (%s)" % (
                r["cpu_baseline"]["value"], r["cpu_baseline"]["unit"], threads,
                r["cpu_baseline"]["sample"]), file=sys.stderr, flush=True)
        results[name] = r
        del w
    head = results[HEADLINE]
    cpu = None if a.no_cpu_baseline else cpu_baseline(workloads, a.cpu_seconds)
    ceil = None if a.quick else ceilings(torch, dev)
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
                     "frac": round(head["frac"], 4), "traffic": head["traffic"],
                     "bytes_per_launch": head["work_per_call"]},
        "cpu_baseline": None if cpu is None else {k: (round(v, 4) if isinstance(v, float) else v)
                                                  for k, v in cpu.items()},
        "ceilings": ceil,
        "workloads": {n: _rounded(r) for n, r in results.items()},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
