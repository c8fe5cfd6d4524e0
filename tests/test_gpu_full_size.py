"""Full-size parity on the five workloads: every key, every decision.

Each workload is quantized at its full size in one call, scored and
reconstructed on the GPU as the bench launches it; the oracle then runs over
the whole cache in chunks of keys and every code, sign, norm and rho is
compared (``oracle.parity.compare_quantize``).  The mismatch counts are
summed over all elements and the rate is asserted below 1e-5 of them.
Scores are compared for every key against the first ``score_queries``
queries of each group (all queries for the KV-cache workloads, 256 for the
search and cone workloads: the oracle's fp64 scores of 1e4 queries x 1e6
keys would take hours); every key's stage-1 reconstruction from the full
grid launch is compared with the oracle's reconstruction of the library's
own codes and norms.

Inputs come from ``vector_quantization_quantize_amd.workloads`` (seeded);
expected values only from ``oracle``.
"""
import sys
import time

import numpy as np
import pytest

from oracle import params as P
from oracle import parity
from oracle import tq

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import vector_quantization_quantize_amd as tqm
    from vector_quantization_quantize_amd import workloads as wl
    return torch, tqm, wl


FIELDS = ("elements", "code_mismatch", "code_bad", "sign_mismatch", "sign_bad", "sign_bad_normalized",
          "cascade_keys", "decision_keys", "norm_bad", "rnorm_bad", "padding_bad")


def full_check(env, name, score_queries=None, chunk=65536, strict_signs=True):
    """Quantize, score and reconstruct workload `name` at full size on the
    GPU; compare every key with the oracle in chunks.  Returns the summed
    counts.  strict_signs=False asserts the sign window |p| / sqrt(d) < 1e-6
    instead of |p| < 1e-6 (the strict count is still printed)."""
    torch, tqm, wl = env
    w = wl.WORKLOADS[name]
    nqs = w.nq if score_queries is None else min(score_queries, w.nq)
    _announce(f"{name} full size: keys={w.total_keys} d={w.d} bits={w.bits} groups={w.groups} "
              f"score queries={nqs} of {w.nq} per group")
    t0 = time.time()
    keys = wl.keys(w, 0)
    queries = wl.queries(w, 0)[:, :nqs]
    h = tqm.tq_init(w.d, w.bits, 0)
    pr = P.init(w.d, w.bits, 0)
    kd = torch.from_numpy(keys).to(torch.bfloat16 if w.key_dtype == "bf16" else torch.float32).cuda()
    codes, signs, norms, rnorms = tqm.tq_quantize(h, kd)
    del kd
    scores = tqm.tq_logits(h, torch.from_numpy(np.ascontiguousarray(queries)).cuda(), codes, signs, norms, rnorms,
                           n=w.n)
    khat = tqm.tq_dequant_mse(h, codes, norms)
    torch.cuda.synchronize()
    print(f"  GPU done in {time.time() - t0:.1f} s", flush=True)
    step = min(chunk, w.n)
    total = {f: 0 for f in FIELDS}
    worst_score = worst_dq = 0.0
    for g in range(w.groups):
        for t0_ in range(0, w.n, step):
            lo = g * w.n + t0_
            hi = lo + min(step, w.n - t0_)
            qz = tq.quantize(pr, keys[lo:hi].astype(np.float64))
            c, s, nn, rr = (x[lo:hi].cpu().numpy() for x in (codes, signs, norms, rnorms))
            rep = parity.compare_quantize(pr, qz, c, s, nn, rr)
            for f in FIELDS:
                total[f] += getattr(rep, f)
            ref = rep.reference
            sref = parity.e2e_scores(pr, rep, queries[g], qz.norms)
            bad, worst = parity.score_violations(scores[g, :, t0_:t0_ + hi - lo].cpu().numpy(), sref, queries[g],
                                                 qz.norms)
            assert bad == 0, (name, g, t0_, "scores", bad, worst)
            worst_score = max(worst_score, worst)
            kref = tq.dequant_mse(pr, ref.idx, nn.astype(np.float64))
            bad, worst = parity.dequant_violations(khat[lo:hi].cpu().numpy(), kref)
            assert bad == 0, (name, g, t0_, "reconstruction", bad, worst)
            worst_dq = max(worst_dq, worst)
    rate = (total["code_mismatch"] + total["sign_mismatch"]) / total["elements"]
    print(f"  {name}: {total}; mismatch rate {rate:.3g}; worst score error {worst_score:.3g} of tolerance; "
          f"worst reconstruction error {worst_dq:.3g} of tolerance; {time.time() - t0:.1f} s", flush=True)
    for f in ("code_bad", "sign_bad" if strict_signs else "sign_bad_normalized", "norm_bad", "rnorm_bad",
              "padding_bad"):
        assert total[f] == 0, (name, total)
    assert rate < parity.MISMATCH_RATE, (name, total)
    tqm.tq_destroy(h)
    return total


@pytest.mark.timeout(300)
def test_toy_every_key(env):
    full_check(env, "toy")


@pytest.mark.timeout(300)
def test_llama_decode_every_key(env):
    full_check(env, "llama_decode")


@pytest.mark.timeout(600)
def test_long_context_every_key(env):
    full_check(env, "long_context")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["search_b2", "search_b4"])
def test_search_every_key(env, name):
    full_check(env, name, score_queries=256)


@pytest.mark.timeout(900)
def test_cone_every_key(env):
    full_check(env, "cone", score_queries=256, chunk=16384)
