"""Throughput of the TurboQuant quantize / score path on one MI355X.

One step = the whole path over one batch of the long-context workload
(batch 4 x 8 KV heads x 131072 bf16 keys, d = 128, 3 bits, 32 query heads per
batch entry, 4 per KV head):
  tq_quantize     the full key cache -> packed codes, signs, norms
  tq_logits       every query head against its KV head's packed keys
  tq_dequant_mse  stage-1 reconstruction of the full cache
All inputs are synthetic (seeded), resident in HBM before timing starts.

Prints one JSON line.  ``value`` = (query, key) scores produced per second of
step time.  Per-kernel times come from HIP events recorded on the stream the
library launches on; ``roofline`` is for the kernel with the largest share of
the step.  ``cpu_baseline`` times the CPU oracle on a bounded sample of the
same workload on the host cores.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "tq_logits keys scored/s + % HBM roofline (d=128, 3-bit); tq_quantize Mkeys/s"
HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
FP32_VALU_PEAK_TFLOPS = 157.3


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="long_context")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cold-reps", type=int, default=10, help="flushed-cache reps per kernel")
    ap.add_argument("--cpu-groups", type=int, default=24, help="key groups timed on the CPU oracle")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-search", action="store_true", help="skip the search (top-k) measurement")
    ap.add_argument("--search-workload", default="search_b2")
    ap.add_argument("--no-split", action="store_true",
                    help="skip the fractional-width line (2.5 and 3.5 bits, general kernels)")
    ap.add_argument("--no-attention", action="store_true",
                    help="skip the decode-attention and uncompressed-logits measurement")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    return ap.parse_args()


def copy_calibration():
    """A plain device-to-device copy of exactly 1 GiB, five times: under
    rocprofv3 --pmc its FETCH_SIZE / WRITE_SIZE per dispatch give the factor
    between counter readings and bytes moved."""
    import torch
    torch.cuda.set_device(0)
    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": nbytes, "copy_calibration_bytes_written": nbytes,
                      "dispatches": 5}), flush=True)


def kernel_models(w):
    """Algorithmic bytes / flops per key of each entry point (see the roofline
    table in the design notes): packed bytes = 4 B W + 4 W + 8."""
    words = (w.d + 31) // 32
    packed = 4 * (w.bits - 1) * words + 4 * words + 8
    key_in = w.d * (2 if w.key_dtype == "bf16" else 4)
    return {
        "tq_quantize": {"bytes": key_in + packed, "flops": 4 * w.d * w.d},
        "tq_logits": {"bytes": packed + 4 * w.nq, "flops": 4 * w.d * w.nq},
        "tq_dequant_mse": {"bytes": 4 * (w.bits - 1) * words + 4 + 4 * w.d, "flops": 2 * w.d * w.d},
    }


def measured_profile(workload):
    """From the committed rocprofv3 summary, for every kernel whose source is
    unchanged since it was taken: HBM bytes per launch (FETCH_SIZE and
    WRITE_SIZE, calibrated) and the matrix cores' busy share of its cycles."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    traffic, mfma_busy = {}, {}
    if not os.path.exists(path):
        return traffic, mfma_busy
    for line in open(path):
        if line.startswith("#") or not line.strip():
            continue
        fields = dict(f.split("=", 1) for f in line.split()[1:])
        entry = line.split()[0]
        src = os.path.join(ROOT, fields["source"])
        if os.path.exists(src) and hashlib.sha1(open(src, "rb").read()).hexdigest() == fields["sha1"]:
            traffic[entry] = int(float(fields["fetch_bytes"]) + float(fields["write_bytes"]))
            if "mfma_busy_pct" in fields:
                mfma_busy[entry] = float(fields["mfma_busy_pct"])
    return traffic, mfma_busy


def search_topk(name, seed, k=10, reps=3, recall_queries=64):
    """Top-k search over a full search workload (every query against every
    key, best k per query, no score matrix): time per call and recall of
    the returned keys against the exact inner products of the unquantized
    vectors on a sample of queries (plain numpy brute force)."""
    import numpy as np
    import torch

    import vector_quantization_quantize_amd as tqm
    from vector_quantization_quantize_amd import workloads as wl
    w = wl.WORKLOADS[name]
    keys_np = wl.keys(w, seed)
    queries_np = wl.queries(w, seed)
    h = tqm.tq_init(w.d, w.bits, 0)
    keys = torch.from_numpy(keys_np).cuda()
    queries = torch.from_numpy(queries_np).cuda()
    packed = tqm.tq_quantize(h, keys)
    del keys
    ws = torch.empty(tqm.tq_logits_topk_workspace_size(h, w.groups, w.nq, w.n, k) // 4 + 64, dtype=torch.float32,
                     device="cuda")
    out = (torch.empty((w.groups, w.nq, k), dtype=torch.int64, device="cuda"),
           torch.empty((w.groups, w.nq, k), dtype=torch.float32, device="cuda"))
    fn = lambda: tqm.tq_logits_topk(h, queries, *packed, k=k, n=w.n, out=out, workspace=ws)
    fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    found = out[0][0, :recall_queries].cpu().numpy()
    sample = queries_np[0, :recall_queries].astype(np.float64)
    exact = sample @ keys_np.astype(np.float64).T
    top = np.argsort(-exact, axis=1, kind="stable")[:, :k]
    recall = float(np.mean([len(set(f) & set(t)) / k for f, t in zip(found.tolist(), top.tolist())]))
    recall1 = float(np.mean([t[0] in set(f) for f, t in zip(found.tolist(), top.tolist())]))
    scores = w.groups * w.nq * w.n
    kp = (w.d + 15) // 16 * 16
    # algorithmic work per score: d level products and d signed adds (4d
    # flops); the matrix-core scorer runs f16 passes over K = d rounded up
    # to 16: one for the signs plus one for the level values when they fit
    # one float16 piece (one or two index bits), two otherwise
    passes = 2 if w.bits <= 3 else 3
    useful = 4.0 * w.d * scores / (ms * 1e-3) / 1e12
    raw = passes * 2.0 * kp * scores / (ms * 1e-3) / 1e12
    tqm.tq_destroy(h)
    return {"workload": f"{w.name}: {w.description}", "keys": w.n * w.groups, "queries": w.nq * w.groups, "d": w.d,
            "bits": w.bits, "k": k, "ms": round(ms, 3), "scores_per_s": scores / (ms * 1e-3),
            "recall_at_10": round(recall, 4), "recall_1_at_10": round(recall1, 4),
            "recall_sample_queries": recall_queries,
            "roofline": {"bound": "mfma", "achieved": round(useful, 2), "peak": BF16_MFMA_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(useful / BF16_MFMA_PEAK_TFLOPS, 4),
                         "raw_mfma_TFLOPs": round(raw, 2)}}


def attention_leg(w, h, keys, queries, packed, seed, stream, reps=10):
    """Decode attention over the compressed cache of the step's workload and
    the uncompressed comparison.  Values: seeded N(0,1) bfloat16 vectors
    quantized with their own handle (same bits, seed 1) and regrouped into
    token blocks; every query head attends over its KV head's n tokens with
    scale 1/sqrt(d).  Comparison: inner products of the same queries with
    the unquantized keys, as float32 and as bfloat16.  Times: HIP events on
    the library's stream, mean of `reps` calls after one warm-up."""
    import torch

    import vector_quantization_quantize_amd as tqm
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1000 + seed)
    values = torch.randn((w.total_keys, w.d), generator=gen, device="cuda").to(torch.bfloat16)
    hv = tqm.tq_init(w.d, w.bits, 1)
    vc, vs, vn, vr = tqm.tq_quantize(hv, values, stream=stream)
    del values, vs, vr
    vblocks = tqm.tq_pack_values(hv, vc, groups=w.groups, n=w.n, stream=stream)
    del vc
    out = torch.empty((w.groups, w.nq, w.d), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.groups, w.nq), dtype=torch.float32, device="cuda")
    ws = torch.empty(tqm.tq_attention_workspace_size(h, hv, w.groups, w.nq, w.n) // 4 + 64, dtype=torch.float32,
                     device="cuda")
    scores = torch.empty((w.groups, w.nq, w.n), dtype=torch.float32, device="cuda")
    lws = torch.empty(tqm.tq_logits_workspace_size(h, w.groups, w.nq) // 4 + 64, dtype=torch.float32,
                      device="cuda")

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    t_attn = timed(lambda: tqm.tq_attention(h, hv, queries, *packed, vblocks, vn, n=w.n, out=out, lse=lse,
                                            workspace=ws, stream=stream))
    t_logits = timed(lambda: tqm.tq_logits(h, queries, *packed, n=w.n, scores=scores, workspace=lws,
                                           stream=stream))
    kb = keys.to(torch.bfloat16) if keys.dtype != torch.bfloat16 else keys
    kf = keys.float()
    t_f32 = timed(lambda: tqm.tq_dense_logits(queries, kf, n=w.n, scores=scores, stream=stream))
    del kf
    t_bf16 = timed(lambda: tqm.tq_dense_logits(queries, kb, n=w.n, scores=scores, stream=stream))
    tokens = w.total_keys
    words = (w.d + 31) // 32
    key_bytes = 4 * (w.bits - 1) * words + 4 * words + 8
    value_bytes = 4 * (w.bits - 1) * words + 4
    # algorithmic bytes: the packed keys and values once (scores, in the
    # ideal, never leave the chip) plus the outputs
    alg = (key_bytes + value_bytes) * tokens + 4 * w.groups * w.nq * (w.d + 1)
    gbs = alg / (t_attn * 1e-3) / 1e9
    dense_b = {"f32": 4 * w.d, "bf16": 2 * w.d}
    res = {"ms": round(t_attn, 4), "ms_scores": round(t_logits, 4), "ms_values": round(t_attn - t_logits, 4),
           "tokens_per_s": tokens / (t_attn * 1e-3), "bytes_per_token": key_bytes + value_bytes,
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(gbs / HBM_PEAK_GBS, 4)},
           "value_bits": w.bits - 1, "scale": "1/sqrt(d)",
           "dense_logits": {}}
    for name, t in (("f32", t_f32), ("bf16", t_bf16)):
        b = (dense_b[name] + 4 * w.nq) * tokens
        res["dense_logits"][name] = {"ms": round(t, 4), "GBps": round(b / (t * 1e-3) / 1e9, 1),
                                     "tq_logits_speedup": round(t / t_logits, 2)}
    tqm.tq_destroy(hv)
    return res


def dequant_prod_leg(w, h, packed, out, stream, reps=10):
    """The reconstruction with the QJL correction (tq_dequant_prod) over the
    step's packed cache into the step's reconstruction buffer: time per call
    (mean of `reps` after a warm-up) against HBM, algorithmic bytes per key =
    packed codes + sign bits + norm + residual norm read, 4 d float32
    written; the 4 d^2 flops per key (G^T s, then Pi^T t) are reported
    beside it."""
    import torch

    import vector_quantization_quantize_amd as tqm
    fn = lambda: tqm.tq_dequant_prod(h, *packed, ktilde=out, stream=stream)
    fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    tfl = 4.0 * w.d * w.d * w.total_keys / (ms * 1e-3) / 1e12
    nbytes = sum(t.numel() * t.element_size() for t in packed) + 4 * w.d * w.total_keys
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"ms": round(ms, 3), "keys": w.total_keys, "TFLOPs": round(tfl, 2),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_key": nbytes / w.total_keys}}


def split_leg(w, keys, queries, scores, khat, seed, stream, reps=3):
    """Fractional widths (tq_init_split) on the step's keys and queries: the
    first d/2 rotated coordinates with one more index bit, 2.5 and 3.5 bits
    per coordinate with the sign bit.  Per width: tq_quantize, tq_logits and
    tq_dequant_mse (general float32 kernels: the matrix-core paths take one
    width only), mean of `reps` calls after a warm-up, and the packed bytes
    per key against the plain handles'."""
    import torch

    import vector_quantization_quantize_amd as tqm

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    res = {}
    hi = w.d // 2
    for bits in (2, 3):
        h = tqm.tq_init_split(w.d, bits, hi, seed)
        packed = tqm.empty_packed(h, w.total_keys)
        lws = torch.empty(tqm.tq_logits_workspace_size(h, w.groups, w.nq) // 4 + 64, dtype=torch.float32,
                          device="cuda")
        t_q = timed(lambda: tqm.tq_quantize(h, keys, out=packed, stream=stream))
        t_l = timed(lambda: tqm.tq_logits(h, queries, *packed, n=w.n, scores=scores, workspace=lws, stream=stream))
        t_d = timed(lambda: tqm.tq_dequant_mse(h, packed[0], packed[2], khat=khat, stream=stream))
        kb = h.layout.key_bytes
        res[f"{bits + hi / w.d:g}_bits"] = {
            "bits": bits, "hi": hi, "key_bytes": kb, "tq_quantize_ms": round(t_q, 3), "tq_logits_ms": round(t_l, 4),
            "tq_dequant_mse_ms": round(t_d, 3),
            "logits_GBps": round((kb * w.total_keys) / (t_l * 1e-3) / 1e9, 1),
            "keys_scored_per_s": w.groups * w.nq * w.n / (t_l * 1e-3)}
        del packed, lws
        tqm.tq_destroy(h)
    return res


def decode_leg(seed, reps=50):
    """One decode step at the llama_decode shape (8 key heads x 32768 bf16
    tokens, 4 query heads per key head, d = 128, 4 bits): latency of
    tq_logits, tq_attention (values quantized with their own handle, scale
    1/sqrt(d)) and the uncompressed comparison on the same keys (float32
    and bfloat16).  Mean of `reps` back-to-back calls after a warm-up."""
    import torch

    import vector_quantization_quantize_amd as tqm
    from vector_quantization_quantize_amd import workloads as wl
    w = wl.WORKLOADS["llama_decode"]
    keys = torch.from_numpy(wl.keys(w, seed)).to(torch.bfloat16).cuda()
    values = torch.from_numpy(wl.keys(w, seed + 1)).to(torch.bfloat16).cuda()
    queries = torch.from_numpy(wl.queries(w, seed)).cuda()
    h, hv = tqm.tq_init(w.d, w.bits, 0), tqm.tq_init(w.d, w.bits, 1)
    packed = tqm.tq_quantize(h, keys)
    vc, _, vn, _ = tqm.tq_quantize(hv, values)
    vblocks = tqm.tq_pack_values(hv, vc, groups=w.groups, n=w.n)
    scores = torch.empty((w.groups, w.nq, w.n), dtype=torch.float32, device="cuda")
    lws = torch.empty(tqm.tq_logits_workspace_size(h, w.groups, w.nq) // 4 + 64, dtype=torch.float32, device="cuda")
    out = torch.empty((w.groups, w.nq, w.d), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.groups, w.nq), dtype=torch.float32, device="cuda")
    aws = torch.empty(tqm.tq_attention_workspace_size(h, hv, w.groups, w.nq, w.n) // 4 + 64, dtype=torch.float32,
                      device="cuda")
    kf = keys.float()
    stream = torch.cuda.current_stream()

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps * 1e3

    res = {"workload": f"{w.name}: {w.description}",
           "tq_logits_us": timed(lambda: tqm.tq_logits(h, queries, *packed, n=w.n, scores=scores, workspace=lws)),
           "tq_attention_us": timed(lambda: tqm.tq_attention(h, hv, queries, *packed, vblocks, vn, n=w.n, out=out,
                                                             lse=lse, workspace=aws)),
           "dense_logits_f32_us": timed(lambda: tqm.tq_dense_logits(queries, kf, n=w.n, scores=scores)),
           "dense_logits_bf16_us": timed(lambda: tqm.tq_dense_logits(queries, keys, n=w.n, scores=scores))}
    for k in list(res):
        if k.endswith("_us"):
            res[k] = round(res[k], 2)
    tqm.tq_destroy(h)
    tqm.tq_destroy(hv)
    return res


def cpu_baseline(w, keys_np, queries_np, groups, seed):
    """Oracle (numpy float64) on the first `groups` key groups."""
    import numpy as np
    from oracle import params as P
    from oracle import tq
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    pr = P.init(w.d, w.bits, seed)
    t0 = time.perf_counter()
    scored = 0
    for g in range(groups):
        k = keys_np[g * w.n:(g + 1) * w.n].astype(np.float64)
        qz = tq.quantize(pr, k)
        s = tq.scores(pr, queries_np[g], qz.idx, qz.beta, qz.norms, qz.rnorms)
        tq.dequant_mse(pr, qz.idx, qz.norms)
        scored += s.size
    dt = time.perf_counter() - t0
    return {"value": scored / dt, "unit": "keys scored/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{groups} of {w.groups} key groups ({groups * w.n} keys x {w.nq} queries): quantize + "
                      f"score + stage-1 reconstruction in numpy float64, {dt:.1f} s; cores = BLAS threads "
                      f"(elementwise numpy runs on one)"}


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(keys shard by KV head with no exchange; see the design notes)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import vector_quantization_quantize_amd as tqm
    from vector_quantization_quantize_amd import workloads as wl

    torch.cuda.set_device(0)
    w = wl.WORKLOADS[args.workload]
    keys_np = wl.keys(w, args.seed)
    queries_np = wl.queries(w, args.seed)
    kdtype = torch.bfloat16 if w.key_dtype == "bf16" else torch.float32
    keys = torch.from_numpy(keys_np).to(kdtype).cuda()
    queries = torch.from_numpy(queries_np).cuda()
    h = tqm.tq_init(w.d, w.bits, 0)
    total = w.total_keys
    packed = tqm.empty_packed(h, total)
    scores = torch.empty((w.groups, w.nq, w.n), dtype=torch.float32, device="cuda")
    ws = torch.empty(tqm.tq_logits_workspace_size(h, w.groups, w.nq) // 4 + 64, dtype=torch.float32,
                     device="cuda")
    khat = torch.empty((total, w.d), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    names = ("tq_quantize", "tq_logits", "tq_dequant_mse")

    def calls():
        return (lambda: tqm.tq_quantize(h, keys, out=packed, stream=stream),
                lambda: tqm.tq_logits(h, queries, *packed, n=w.n, scores=scores, workspace=ws, stream=stream),
                lambda: tqm.tq_dequant_mse(h, packed[0], packed[2], khat=khat, stream=stream))

    fns = calls()
    for _ in range(args.warmup):
        for f in fns:
            f()
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in names]
          for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record(stream)
    for s in range(args.steps):
        for i, f in enumerate(fns):
            ev[s][i][0].record(stream)
            f()
            ev[s][i][1].record(stream)
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = start.elapsed_time(stop) / args.steps
    per = {n: float(np.mean([ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(args.steps)]))
           for i, n in enumerate(names)}

    # each kernel again with the caches flushed before every launch: reading
    # 1 GiB (> L2 + MALL) leaves only clean lines behind.  A write-based flush
    # would leave up to the MALL's size of dirty lines whose write-back lands
    # inside the timed kernel and roughly halves its apparent read rate.
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    sink = torch.zeros((), dtype=torch.float32, device="cuda")
    cold = {}
    for i, n in enumerate(names):
        times = []
        for _ in range(args.cold_reps):
            torch.sum(flush, dim=0, out=sink)
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fns[i]()
            b.record(stream)
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        cold[n] = float(np.median(times))
    del flush, sink

    models = kernel_models(w)
    scored = w.groups * w.nq * w.n
    kern = {}
    for n in names:
        units = total  # every entry point processes the whole cache once
        gbs = models[n]["bytes"] * units / (per[n] * 1e-3) / 1e9
        tfl = models[n]["flops"] * units / (per[n] * 1e-3) / 1e12
        gbs_cold = models[n]["bytes"] * units / (cold[n] * 1e-3) / 1e9
        kern[n] = {"ms": round(per[n], 4), "ms_cold": round(cold[n], 4), "GBps": round(gbs, 1),
                   "GBps_cold": round(gbs_cold, 1), "TFLOPs": round(tfl, 2),
                   "bytes_per_key": models[n]["bytes"], "flops_per_key": models[n]["flops"]}
    kern["tq_quantize"]["Mkeys_per_s"] = round(total / (per["tq_quantize"] * 1e-3) / 1e6, 1)
    kern["tq_logits"]["keys_scored_per_s"] = scored / (per["tq_logits"] * 1e-3)
    kern["tq_logits"]["keys_scored_per_s_cold"] = scored / (cold["tq_logits"] * 1e-3)

    # which resource bounds each kernel as built at d = 128: logits streams
    # bytes; quantize runs its two projections on the matrix cores (2 f16
    # passes for Pi k on power-of-two scaled keys + 3 for G r, each 2 d^2, for
    # 4 d^2 useful flops per key); the reconstruction (3 passes of 2 d^2)
    # writes 512 B per key and is bound by HBM writes
    bound = {"tq_quantize": ("mfma", BF16_MFMA_PEAK_TFLOPS), "tq_logits": ("hbm", HBM_PEAK_GBS),
             "tq_dequant_mse": ("hbm", HBM_PEAK_GBS)}
    # reconstruction: 2 passes when the level set has at most two magnitudes
    # (B <= 2 at d = 128), else 3
    raw_passes = {"tq_quantize": 10 * w.d * w.d, "tq_dequant_mse": (4 if w.bits <= 3 else 6) * w.d * w.d}
    for n, f in raw_passes.items():
        kern[n]["raw_mfma_TFLOPs"] = round(f * total / (per[n] * 1e-3) / 1e12, 2)

    def roofline(n):
        kind, peak = bound[n]
        if kind == "hbm":
            ach, ach_cold, unit = kern[n]["GBps"], kern[n]["GBps_cold"], "GB/s"
        else:
            ach, unit = kern[n]["TFLOPs"], "TFLOP/s"
            ach_cold = round(models[n]["flops"] * total / (cold[n] * 1e-3) / 1e12, 2)
        return {"kernel": n, "bound": kind, "achieved": ach, "peak": peak, "unit": unit,
                "frac": round(ach / peak, 4), "traffic": traffic.get(n),
                "achieved_cold": ach_cold, "frac_cold": round(ach_cold / peak, 4),
                "mfma_busy_pct": mfma_busy.get(n)}

    traffic, mfma_busy = measured_profile(args.workload)
    dominant = max(names, key=lambda n: per[n])
    line = {
        "metric": METRIC,
        "value": scored / (step_ms * 1e-3),
        "unit": "keys scored/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.description}", "keys": total, "d": w.d, "bits": w.bits,
                   "queries": w.groups * w.nq, "key_dtype": w.key_dtype,
                   "step": "tq_quantize + tq_logits + tq_dequant_mse over the full cache"},
        "wall_s": round(wall, 3),
        "kernels": kern,
        "roofline": roofline(dominant),
        "roofline_logits": roofline("tq_logits"),
        "roofline_by_kernel": {n: roofline(n) for n in names},
    }
    if not args.no_attention:
        line["attention"] = attention_leg(w, h, keys, queries, packed, args.seed, stream)
        line["decode_step"] = decode_leg(args.seed)
        line["dequant_prod"] = dequant_prod_leg(w, h, packed, khat, stream)
    if not args.no_split:
        line["fractional_widths"] = split_leg(w, keys, queries, scores, khat, args.seed, stream)
    if not args.no_search:
        del keys, queries, packed, scores, ws, khat
        torch.cuda.empty_cache()
        line["search_topk"] = search_topk(args.search_workload, args.seed)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, keys_np, queries_np, min(args.cpu_groups, w.groups), args.seed)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
