"""Throughput of the TurboQuant quantize / score path on one MI355X.

One step = the whole path over one batch of the long-context workload
(batch 4 x 8 KV heads x 131072 bf16 keys, d = 128, 3 bits, 32 query heads per
batch entry, 4 per KV head):
  tq_quantize     the full key cache -> packed codes, signs, norms
  tq_logits       every query head against its KV head's packed keys
  tq_dequant_mse  stage-1 reconstruction of the full cache
All inputs are synthetic (seeded), resident in HBM before timing starts.

Prints one JSON line.  ``value`` = tq_logits (query, key) scores per second,
the kernel timed with cold caches (back-to-back launches rotating over
copies of its inputs that span at least 1 GiB, so every launch reads its
inputs from HBM; the metric's "keys scored/s"); the step's own rate is under
``step``.  Per-kernel times
come from HIP events recorded on the stream the library launches on;
``roofline`` is for the kernel with the largest share of the step, priced
against the roof its arithmetic intensity puts it under.  ``cpu_baseline``
times the CPU oracle on a bounded sample of the same workload on the host
cores, and ``parity`` compares every key of that sample with the GPU's
output from the timed step.
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
    ap.add_argument("--cold-reps", type=int, default=10, help="rounds over the cold-cache input copies per kernel")
    ap.add_argument("--cpu-groups", type=int, default=24, help="key groups timed on the CPU oracle")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-search", action="store_true", help="skip the search (top-k) measurement")
    ap.add_argument("--search-workload", default="search_b2")
    ap.add_argument("--no-split", action="store_true",
                    help="skip the fractional-width (2.5 and 3.5 bits) and polar-angle lines")
    ap.add_argument("--no-attention", action="store_true",
                    help="skip the decode-attention and uncompressed-logits measurement")
    ap.add_argument("--no-general", action="store_true",
                    help="skip the float32-key quantize line (cone, search, toy)")
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
    """From the committed rocprofv3 summary, for every kernel whose sources
    are unchanged since it was taken: HBM bytes per launch (FETCH_SIZE and
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
        # the kernel's sources (comma-separated), hashed in order as one text
        srcs = [os.path.join(ROOT, f) for f in fields["source"].split(",")]
        if all(os.path.exists(f) for f in srcs) and \
                hashlib.sha1(b"".join(open(f, "rb").read() for f in srcs)).hexdigest() == fields["sha1"]:
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
    the library's stream, mean of `reps` calls after one warm-up; the
    two-kernel form (TQ_ATTN_FUSED=0) is timed on the same inputs beside
    the default one-kernel form."""
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
    # the two-kernel form (scores through the workspace, then the value
    # pass) on the same inputs, for comparison
    os.environ["TQ_ATTN_FUSED"] = "0"
    try:
        t_two = timed(lambda: tqm.tq_attention(h, hv, queries, *packed, vblocks, vn, n=w.n, out=out, lse=lse,
                                               workspace=ws, stream=stream))
    finally:
        del os.environ["TQ_ATTN_FUSED"]
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
    res = {"ms": round(t_attn, 4), "form": "one kernel: scores stay on chip",
           "ms_two_kernel": round(t_two, 4), "ms_logits_alone": round(t_logits, 4),
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


def cold_logits_ms(h, queries, packed, n, scores, ws, stream, rounds=5):
    """tq_logits with cold caches, timed as the headline scorer is: launches
    back to back over R copies of the packed keys and the scores (R copies
    of the packed keys span at least 1 GiB, more than L2 + MALL), HIP events
    on the launch stream around all rounds x R launches.  Returns the time
    per launch (ms) and R."""
    import torch

    import vector_quantization_quantize_amd as tqm
    in_bytes = sum(t.numel() * t.element_size() for t in packed)
    r = max(2, -(-(1 << 30) // in_bytes))
    sets = [(tuple(t.clone() for t in packed), torch.empty_like(scores)) for _ in range(r)]
    run = [lambda p=p, o=o: tqm.tq_logits(h, queries, *p, n=n, scores=o, workspace=ws, stream=stream)
           for p, o in sets]
    for f in run:  # warm-up round
        f()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(rounds):
        for f in run:
            f()
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / (rounds * r)
    del sets, run
    torch.cuda.empty_cache()
    return ms, r


def split_leg(w, keys, queries, scores, khat, seed, stream, reps=3):
    """Fractional widths (tq_init_split) on the step's keys and queries: the
    first d/2 rotated coordinates with one more index bit, 2.5 and 3.5 bits
    per coordinate with the sign bit.  Per width: tq_quantize (the d = 128
    matrix-core quantizer, two waves on the finer level set), tq_logits (the
    byte-table scorer, the two halves in separate byte phases) and
    tq_dequant_mse (matrix cores), mean of `reps` calls after a warm-up,
    and the packed bytes per key against the plain handles'.  tq_logits is
    also timed with cold caches (cold_logits_ms); its GB/s, HBM fraction and
    scoring rate are the cold ones, over the packed bytes read plus the
    scores written."""
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
        t_c, r = cold_logits_ms(h, queries, packed, w.n, scores, lws, stream)
        kb = h.layout.key_bytes
        gbs = (kb + 4 * w.nq) * w.total_keys / (t_c * 1e-3) / 1e9
        res[f"{bits + hi / w.d:g}_bits"] = {
            "bits": bits, "hi": hi, "key_bytes": kb, "tq_quantize_ms": round(t_q, 3), "tq_logits_ms": round(t_l, 4),
            "tq_logits_ms_cold": round(t_c, 4), "cold_copies": r, "tq_dequant_mse_ms": round(t_d, 3),
            "logits_GBps": round(gbs, 1), "logits_hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "keys_scored_per_s": w.groups * w.nq * w.n / (t_c * 1e-3)}
        del packed, lws
        tqm.tq_destroy(h)
    return res


def polar_leg(w, keys, queries, scores, khat, seed, stream, reps=3):
    """The recursive polar-angle stage 1 (tq_init_polar) on the step's keys
    and queries: tq_quantize, tq_logits and tq_dequant_mse per call (mean of
    `reps` after a warm-up), against HBM with the plain handle's packed
    bytes per key (the angle indices fill the same bit planes).  tq_logits's
    HBM fraction and scoring rate are the cold-cache ones (cold_logits_ms)."""
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

    h = tqm.tq_init_polar(w.d, w.bits, seed)
    packed = tqm.empty_packed(h, w.total_keys)
    lws = torch.empty(tqm.tq_logits_workspace_size(h, w.groups, w.nq) // 4 + 64, dtype=torch.float32,
                      device="cuda")
    t_q = timed(lambda: tqm.tq_quantize(h, keys, out=packed, stream=stream))
    t_l = timed(lambda: tqm.tq_logits(h, queries, *packed, n=w.n, scores=scores, workspace=lws, stream=stream))
    t_d = timed(lambda: tqm.tq_dequant_mse(h, packed[0], packed[2], khat=khat, stream=stream))
    t_c, r = cold_logits_ms(h, queries, packed, w.n, scores, lws, stream)
    kb = h.layout.key_bytes
    n = w.total_keys
    qb = (w.d * keys.element_size() + kb) * n
    lb = (kb + 4 * w.nq) * n
    db = (kb - 4 * ((w.d + 31) // 32) - 4 + 4 * w.d) * n
    res = {"bits": w.bits, "key_bytes": kb,
           "tq_quantize_ms": round(t_q, 3), "quantize_hbm_frac": round(qb / (t_q * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "tq_logits_ms": round(t_l, 4), "tq_logits_ms_cold": round(t_c, 4), "cold_copies": r,
           "logits_hbm_frac": round(lb / (t_c * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "keys_scored_per_s": w.groups * w.nq * w.n / (t_c * 1e-3),
           "tq_dequant_mse_ms": round(t_d, 3), "dequant_hbm_frac": round(db / (t_d * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "kernels": "d = 128: quantize_polar128_kernel (matrix-core rotation and projection, angle "
                      "recursion in registers), logits_polar128_kernel (byte tables), dequant_polar128_kernel "
                      "(matrix cores); other d: float32 vector kernels"}
    del packed, lws
    tqm.tq_destroy(h)
    return res


def toy_leg(seed, reps=50):
    """The toy workload (4096 float32 keys, d = 128, 3 bits, 16 queries):
    latency of tq_quantize and tq_logits, mean of `reps` back-to-back calls
    after a warm-up (inputs stay in cache at this size)."""
    import torch

    import vector_quantization_quantize_amd as tqm
    from vector_quantization_quantize_amd import workloads as wl
    w = wl.WORKLOADS["toy"]
    keys = torch.from_numpy(wl.keys(w, seed)).cuda()
    queries = torch.from_numpy(wl.queries(w, seed)).cuda()
    h = tqm.tq_init(w.d, w.bits, 0)
    packed = tqm.tq_quantize(h, keys)
    scores = torch.empty((w.groups, w.nq, w.n), dtype=torch.float32, device="cuda")
    lws = torch.empty(tqm.tq_logits_workspace_size(h, w.groups, w.nq) // 4 + 64, dtype=torch.float32, device="cuda")
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
        return round(a.elapsed_time(b) / reps * 1e3, 2)

    return {"workload": f"{w.name}: {w.description}",
            "tq_quantize_us": timed(lambda: tqm.tq_quantize(h, keys, out=packed)),
            "tq_logits_us": timed(lambda: tqm.tq_logits(h, queries, *packed, n=w.n, scores=scores, workspace=lws))}


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
           "tq_quantize_us": timed(lambda: tqm.tq_quantize(h, keys, out=packed)),
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


def _host_cores():
    """Cores this process may run on (its CPU affinity)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def quantize_general_leg(seed, reps=5):
    """tq_quantize on the float32-key workloads (the general matrix-core
    quantizer: norms and key pieces, then Z = Pi K and P = G R as tiled
    f16 matrix-core products with operands split into two pieces): cone
    (1e6 x 1536, 4 bits), search_b2 / search_b4 (1e6 x 200) and toy.  Keys
    are drawn on the device with the workload's law (the search and toy
    generators' exact streams are not needed for timing).  Per workload:
    ms per call (mean of `reps` after a warm-up), Mkeys/s, HBM GB/s of keys
    in + packed out, useful matrix flops (4 d^2 per key) and raw matrix
    flops (3 passes of 2 x 128-row tiles x K for Z = Pi K, 2 for P = G R
    with the seeded float16-exact G; rows of 32 per bit word instead of 128
    per tile where the one-kernel quantizer runs, 16 <= d <= 208 with d a
    multiple of 8) against the bf16 matrix-core peak."""
    import numpy as np
    import torch

    import vector_quantization_quantize_amd as tqm
    from vector_quantization_quantize_amd import workloads as wl
    gen = torch.Generator(device="cuda")
    gen.manual_seed(2000 + seed)
    res = {}
    for name in ("cone", "search_b2", "search_b4", "toy"):
        w = wl.WORKLOADS[name]
        n, d = w.total_keys, w.d
        if name == "cone":
            mu, basis = wl._cone_frame(w, seed)
            mu_t = torch.from_numpy(mu).float().cuda()
            b_t = torch.from_numpy(basis).float().cuda()
            keys = torch.empty((n, d), dtype=torch.float32, device="cuda")
            for c0 in range(0, n, 1 << 16):
                m = min(1 << 16, n - c0)
                z = torch.randn((m, 64), generator=gen, device="cuda")
                eps = 0.01 * torch.randn((m, d), generator=gen, device="cuda")
                x = 0.87 * mu_t[None, :] + 0.49 * (z @ b_t.T / 8.0 + eps)
                keys[c0:c0 + m] = x / x.norm(dim=1, keepdim=True)
        elif name.startswith("search"):
            scale = torch.arange(1, d + 1, device="cuda", dtype=torch.float32) ** -0.5
            keys = torch.randn((n, d), generator=gen, device="cuda") * scale[None, :]
            keys /= keys.norm(dim=1, keepdim=True)
        else:
            keys = torch.from_numpy(wl.keys(w, seed)).cuda()
        h = tqm.tq_init(d, w.bits, 0)
        out = tqm.empty_packed(h, n)
        fn = lambda: tqm.tq_quantize(h, keys, out=out)
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        words = (d + 31) // 32
        dpm = 32 * words
        kp = (d + 15) // 16 * 16
        nct = (dpm + 127) // 128
        packed = 4 * (w.bits - 1) * words + 4 * words + 8
        useful = 4.0 * d * d * n / (ms * 1e-3) / 1e12
        one_kernel = 16 <= d <= 208 and d % 8 == 0
        rows = dpm if one_kernel else 128 * nct
        raw = 2.0 * rows * (3 * kp + 2 * dpm) * n / (ms * 1e-3) / 1e12
        gbs = (4 * d + packed) * n / (ms * 1e-3) / 1e9
        res[name] = {"keys": n, "d": d, "bits": w.bits, "ms": round(ms, 3), "Mkeys_per_s": round(n / ms / 1e3, 1),
                     "kernel": "one-kernel quantizer" if one_kernel else "tiled general quantizer",
                     "GBps": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                     "useful_TFLOPs": round(useful, 1), "useful_mfma_frac": round(useful / BF16_MFMA_PEAK_TFLOPS, 4),
                     "raw_TFLOPs": round(raw, 1), "raw_mfma_frac": round(raw / BF16_MFMA_PEAK_TFLOPS, 4)}
        tqm.tq_destroy(h)
        del keys, out
        torch.cuda.empty_cache()
    # a randomized Hadamard handle against a Haar handle on the same 1e6
    # unit keys of a power-of-two d: fast transform + projection versus the
    # two dense products
    n, d = 1000000, 1024
    keys = torch.randn((n, d), generator=gen, device="cuda")
    keys /= keys.norm(dim=1, keepdim=True)
    had = {"keys": n, "d": d, "bits": 4}
    for kind, init in (("haar", tqm.tq_init), ("hadamard", tqm.tq_init_hadamard)):
        h = init(d, 4, 0)
        out = tqm.empty_packed(h, n)
        tqm.tq_quantize(h, keys, out=out)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            tqm.tq_quantize(h, keys, out=out)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        had[kind + "_ms"] = round(ms, 3)
        had[kind + "_GBps"] = round((4 * d + 4 * 4 * (d // 32) + 8) * n / (ms * 1e-3) / 1e9, 1)
        tqm.tq_destroy(h)
        del out
    res["hadamard_d1024"] = had
    del keys
    torch.cuda.empty_cache()
    c = res["cone"]
    res["roofline_cone"] = {"bound": "mfma", "achieved": c["useful_TFLOPs"], "peak": BF16_MFMA_PEAK_TFLOPS,
                            "unit": "TFLOP/s", "frac": c["useful_mfma_frac"], "raw_frac": c["raw_mfma_frac"],
                            "note": "useful = 4 d^2 flops per key (the two projections); raw = the f16 passes run"}
    return res


def cpu_baseline(w, keys_np, queries_np, groups, seed, gpu_out):
    """Oracle (numpy float64) on the first `groups` key groups, timed on the
    host cores with BLAS limited to the process's CPU affinity; then (not
    timed) every key of those groups compared with the GPU's packed output,
    scores and reconstruction from the timed step (``gpu_out``: codes,
    signs, norms, rnorms, scores, khat as device tensors)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import params as P
    from oracle import parity
    from oracle import tq
    cores = _host_cores()
    pr = P.init(w.d, w.bits, seed)
    fields = ("elements", "code_mismatch", "code_bad", "sign_mismatch", "sign_bad", "sign_bad_normalized",
              "cascade_keys", "decision_keys", "norm_bad", "rnorm_bad", "padding_bad")
    total = {f: 0 for f in fields}
    bad_scores = bad_khat = 0
    worst_score = worst_khat = 0.0
    codes, signs, norms, rnorms, scores, khat = gpu_out
    dt = 0.0
    scored = 0
    with threadpool_limits(limits=cores):
        for g in range(groups):
            sl = slice(g * w.n, (g + 1) * w.n)
            k = keys_np[sl].astype(np.float64)
            t0 = time.perf_counter()
            qz = tq.quantize(pr, k)
            s = tq.scores(pr, queries_np[g], qz.idx, qz.beta, qz.norms, qz.rnorms)
            kh = tq.dequant_mse(pr, qz.idx, qz.norms)
            dt += time.perf_counter() - t0
            scored += s.size
            # parity of this group (outside the timed region)
            nn = norms[sl].cpu().numpy()
            rep = parity.compare_quantize(pr, qz, codes[sl].cpu().numpy(), signs[sl].cpu().numpy(), nn,
                                          rnorms[sl].cpu().numpy())
            for f in fields:
                total[f] += getattr(rep, f)
            ref = rep.reference
            if rep.decision_keys:
                s = parity.e2e_scores(pr, rep, queries_np[g], qz.norms)
            b, wr = parity.score_violations(scores[g].cpu().numpy(), s, queries_np[g], qz.norms)
            bad_scores += b
            worst_score = max(worst_score, wr)
            kh = tq.dequant_mse(pr, ref.idx, nn.astype(np.float64))
            b, wr = parity.dequant_violations(khat[sl].cpu().numpy(), kh)
            bad_khat += b
            worst_khat = max(worst_khat, wr)
        # the toy workload on one thread: the oracle's single-core rate
        toy = wl_toy()
        tk, tqq = toy
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            prt = P.init(128, 3, seed)
            qt = tq.quantize(prt, tk.astype(np.float64))
            st = tq.scores(prt, tqq[0], qt.idx, qt.beta, qt.norms, qt.rnorms)
            tq.dequant_mse(prt, qt.idx, qt.norms)
            dt1 = time.perf_counter() - t0
    rate = (total["code_mismatch"] + total["sign_mismatch"]) / max(total["elements"], 1)
    parity_line = dict(total, mismatch_rate=rate, score_violations=bad_scores, worst_score_error_of_tol=worst_score,
                       reconstruction_violations=bad_khat, worst_reconstruction_error_of_tol=worst_khat,
                       keys_compared=groups * w.n,
                       rule="codes and signs bit-exact outside |z - t| < 1e-6 and |p| < 1e-6, mismatches "
                            "< 1e-5 of all decisions; scores within 1e-3 ||q|| n; reconstruction within 1e-5")
    base = {"value": scored / dt, "unit": "keys scored/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{groups} of {w.groups} key groups ({groups * w.n} keys x {w.nq} queries): quantize + "
                      f"score + stage-1 reconstruction in numpy float64, {dt:.1f} s; BLAS limited to the "
                      f"{cores} cores of the process's CPU affinity (elementwise numpy runs on one)",
            "one_thread_toy": {"value": st.size / dt1, "unit": "keys scored/s", "cores": 1,
                               "sample": f"toy workload (4096 fp32 keys x 16 queries, d = 128, 3 bits), {dt1:.2f} s"}}
    return base, parity_line


def wl_toy():
    from vector_quantization_quantize_amd import workloads as wl
    w = wl.WORKLOADS["toy"]
    return wl.keys(w), wl.queries(w)


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

    # each kernel again with cold caches: launches run back to back over R
    # copies of the kernel's inputs and outputs, R chosen so that the copies
    # of the inputs span at least 1 GiB (> L2 + MALL); a launch's inputs were
    # last touched R - 1 launches (>= 1 GiB of traffic) earlier, so they
    # come from HBM.  HIP events bracket the whole run of R x cold_reps
    # launches on the launch stream; the cold time is that span over the
    # launch count (a single launch bracketed by events would also count
    # the event and dispatch latency around it).
    in_bytes = {"tq_quantize": keys.numel() * keys.element_size(),
                "tq_logits": sum(t.numel() * t.element_size() for t in packed),
                "tq_dequant_mse": packed[0].numel() * 4 + packed[2].numel() * 4}
    cold, cold_copies = {}, {}
    for i, n in enumerate(names):
        r = max(2, -(-(1 << 30) // in_bytes[n]))
        cold_copies[n] = r
        if n == "tq_quantize":
            sets = [(keys.clone(), tqm.empty_packed(h, total)) for _ in range(r)]
            run = [lambda k=k, o=o: tqm.tq_quantize(h, k, out=o, stream=stream) for k, o in sets]
        elif n == "tq_logits":
            sets = [(tuple(t.clone() for t in packed), torch.empty_like(scores)) for _ in range(r)]
            run = [lambda p=p, o=o: tqm.tq_logits(h, queries, *p, n=w.n, scores=o, workspace=ws, stream=stream)
                   for p, o in sets]
        else:
            sets = [((packed[0].clone(), packed[2].clone()), torch.empty_like(khat)) for _ in range(r)]
            run = [lambda p=p, o=o: tqm.tq_dequant_mse(h, p[0], p[1], khat=o, stream=stream) for p, o in sets]
        for f in run:  # warm-up round
            f()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(args.cold_reps):
            for f in run:
                f()
        b.record(stream)
        torch.cuda.synchronize()
        cold[n] = a.elapsed_time(b) / (args.cold_reps * r)
        del sets, run
        torch.cuda.empty_cache()

    # a streaming floor for tq_logits in the same run and the same cold
    # rotation: a plain device copy (the runtime's copy kernel) that moves as
    # many bytes as tq_logits does (packed inputs read + scores written),
    # half read and half written
    moved = in_bytes["tq_logits"] + scores.numel() * scores.element_size()
    half = (moved // 2 + 15) // 16 * 16
    r = max(2, -(-(1 << 30) // half))
    srcs = [torch.ones(half, dtype=torch.uint8, device="cuda") for _ in range(r)]
    dsts = [torch.empty(half, dtype=torch.uint8, device="cuda") for _ in range(r)]
    with torch.cuda.stream(stream):
        for x, y in zip(srcs, dsts):  # warm-up round
            y.copy_(x)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(args.cold_reps):
            for x, y in zip(srcs, dsts):
                y.copy_(x)
        b.record(stream)
        torch.cuda.synchronize()
    floor_ms = a.elapsed_time(b) / (args.cold_reps * r)
    floor_bytes = 2 * half
    del srcs, dsts
    torch.cuda.empty_cache()

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

    # which roof bounds each kernel, by its arithmetic intensity against the
    # ridge of HBM and bf16 matrix cores (2500 TFLOP/s / 8 TB/s = 312 flop/B):
    # quantize does 4 d^2 useful flops on 2 d + 56 bytes per key at d = 128
    # (210 flop/B), logits streams 72 bytes per key for 4 queries, and the
    # reconstruction writes 4 d bytes per key; all three are HBM-bound.  The
    # matrix-core work each one really runs is reported beside it: quantize
    # runs 2 f16 passes for Pi k on power-of-two scaled keys + 2 for G r
    # (G's entries are float16-exact),
    # each 2 d^2 flops; the reconstruction 2 passes when the level set has
    # at most two magnitudes (B <= 2 at d = 128), else 3.
    bound = {n: ("hbm", HBM_PEAK_GBS) for n in names}
    raw_passes = {"tq_quantize": 8 * w.d * w.d, "tq_dequant_mse": (4 if w.bits <= 3 else 6) * w.d * w.d}
    for n, f in raw_passes.items():
        kern[n]["raw_mfma_TFLOPs"] = round(f * total / (per[n] * 1e-3) / 1e12, 2)
        kern[n]["mfma_useful_frac"] = round(kern[n]["TFLOPs"] / BF16_MFMA_PEAK_TFLOPS, 4)
        kern[n]["mfma_raw_frac"] = round(kern[n]["raw_mfma_TFLOPs"] / BF16_MFMA_PEAK_TFLOPS, 4)

    def roofline(n):
        kind, peak = bound[n]
        ach, ach_cold, unit = kern[n]["GBps"], kern[n]["GBps_cold"], "GB/s"
        return {"kernel": n, "bound": kind, "achieved": ach_cold, "peak": peak, "unit": unit,
                "frac": round(ach_cold / peak, 4), "traffic": traffic.get(n),
                "timing": f"cold caches: back-to-back launches over {cold_copies[n]} copies of the inputs "
                          f"(>= 1 GiB apart), HIP events around all {cold_copies[n] * args.cold_reps} launches",
                "achieved_in_step": ach, "frac_in_step": round(ach / peak, 4),
                "bytes_per_key": models[n]["bytes"], "keys_per_launch": total,
                "mfma_busy_pct": mfma_busy.get(n)}

    traffic, mfma_busy = measured_profile(args.workload)
    dominant = max(names, key=lambda n: per[n])
    line = {
        "metric": METRIC,
        "value": scored / (cold["tq_logits"] * 1e-3),
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
                   "step": "tq_quantize + tq_logits + tq_dequant_mse over the full cache",
                   "value": "tq_logits (query, key) scores per second, inputs read from HBM (cold caches)"},
        "step": {"ms": round(step_ms, 4), "keys_scored_per_s": scored / (step_ms * 1e-3),
                 "tq_quantize_Mkeys_per_s": kern["tq_quantize"]["Mkeys_per_s"]},
        "wall_s": round(wall, 3),
        "kernels": kern,
        "roofline": roofline(dominant),
        "roofline_logits": roofline("tq_logits"),
        "roofline_by_kernel": {n: roofline(n) for n in names},
    }
    floor_gbs = floor_bytes / (floor_ms * 1e-3) / 1e9
    line["roofline_logits"]["stream_floor"] = {
        "ms": round(floor_ms, 4), "GBps": round(floor_gbs, 1), "frac": round(floor_gbs / HBM_PEAK_GBS, 4),
        "what": f"plain device copy of {half} bytes (reads {half}, writes {half}: the {floor_bytes} bytes "
                f"tq_logits moves), cold rotation over {r} copies",
        "logits_ms_over_floor_ms": round(cold["tq_logits"] / floor_ms, 3)}
    if not args.no_cpu_baseline:
        line["cpu_baseline"], line["parity"] = cpu_baseline(
            w, keys_np, queries_np, min(args.cpu_groups, w.groups), args.seed,
            (packed[0], packed[1], packed[2], packed[3], scores, khat))
    if not args.no_attention:
        line["attention"] = attention_leg(w, h, keys, queries, packed, args.seed, stream)
        line["decode_step"] = decode_leg(args.seed)
        line["toy"] = toy_leg(args.seed)
        line["dequant_prod"] = dequant_prod_leg(w, h, packed, khat, stream)
    if not args.no_split:
        line["fractional_widths"] = split_leg(w, keys, queries, scores, khat, args.seed, stream)
        line["polar"] = polar_leg(w, keys, queries, scores, khat, args.seed, stream)
    if not args.no_search:
        del keys, queries, packed, scores, ws, khat
        torch.cuda.empty_cache()
        line["search_topk"] = search_topk(args.search_workload, args.seed)
    if not args.no_general:
        torch.cuda.empty_cache()
        line["quantize_general"] = quantize_general_leg(args.seed)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
