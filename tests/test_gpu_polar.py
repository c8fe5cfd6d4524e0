"""Polar-angle stage 1 (tq_init_polar) on the GPU against ``oracle.polar``.

Quantize (angle codes bit-exact outside their level's 1e-6 decision
windows, signs outside |p| < 1e-6, norms and rho), scores of the oracle's
packed keys (decode parity) and of the library's own (end to end against
the oracle's estimator on the library's decisions), the stage-1
reconstruction, the layout, and the entry points that refuse polar handles.
Inputs: seeded numpy draws; expected values only from ``oracle``.
"""
import sys

import numpy as np
import pytest

from oracle import parity
from oracle import polar as PL
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
    return torch, tqm


def _dev(torch, a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def _cpu(t):
    return t.detach().cpu().numpy()


@pytest.mark.parametrize("d,bits,groups,n,nq,key_dtype", [
    (2, 3, 1, 33, 1, "f32"), (4, 3, 1, 50, 2, "f32"), (16, 2, 2, 300, 3, "f32"), (64, 4, 1, 500, 5, "f32"),
    (128, 3, 2, 1000, 4, "bf16"), (128, 2, 3, 777, 5, "f32"), (128, 3, 1, 65, 3, "bf16"), (128, 4, 1, 300, 6, "f32"),
    (128, 5, 1, 999, 4, "bf16"), (128, 2, 1, 20001, 2, "bf16"), (128, 3, 1, 1, 2, "f32"), (128, 4, 2, 31, 3, "bf16"),
    (256, 5, 1, 257, 20, "f32"), (1024, 3, 1, 100, 4, "f32")])
def test_polar_matches_oracle(env, d, bits, groups, n, nq, key_dtype):
    torch, tqm = env
    _announce(f"polar d={d} bits={bits} groups={groups} n={n} nq={nq} {key_dtype}")
    pp = PL.init_polar(d, bits, 9)
    h = tqm.tq_init_polar(d, bits, 9)
    assert h.layout.polar == 1 and h.layout.code_bytes == 4 * (bits - 1) * tq.words_per_plane(d)
    rs = np.random.default_rng(d * 11 + bits)
    keys = rs.standard_normal((groups * n, d)) * np.exp(0.5 * rs.standard_normal((groups * n, 1)))
    keys[min(3, groups * n - 1)] = 0.0      # a zero key runs literally
    if key_dtype == "bf16":
        keys = np.asarray(torch.tensor(keys).bfloat16().float().numpy(), dtype=np.float64)
    queries = rs.standard_normal((groups, nq, d)).astype(np.float32)
    kd = _dev(torch, keys.astype(np.float32), torch.bfloat16 if key_dtype == "bf16" else None)
    codes, signs, norms, rnorms = tqm.tq_quantize(h, kd)
    torch.cuda.synchronize()
    pq = PL.quantize(pp, keys)
    rep = parity.compare_quantize_polar(pp, pq, _cpu(codes), _cpu(signs), _cpu(norms), _cpu(rnorms))
    print(rep.summary())
    assert rep.ok(), rep
    # decode parity: the oracle's packed keys through the library's scorer
    pc = tq.pack_codes(PL.slots(pq.codes), bits - 1)
    ps = tq.pack_bits(pq.beta)
    pn, pr = pq.norms.astype(np.float32), pq.rnorms.astype(np.float32)
    qd = _dev(torch, queries)
    s_dec = _cpu(tqm.tq_logits(h, qd, _dev(torch, pc.view(np.int32)), _dev(torch, ps.view(np.int32)),
                               _dev(torch, pn), _dev(torch, pr), n=n))
    s_e2e = _cpu(tqm.tq_logits(h, qd, codes, signs, norms, rnorms, n=n))
    for g in range(groups):
        sl = slice(g * n, (g + 1) * n)
        ref = PL.scores(pp, queries[g], [c[sl] for c in pq.codes], pq.beta[sl], pn[sl].astype(np.float64),
                        pr[sl].astype(np.float64))
        bad, worst = parity.score_violations(s_dec[g], ref, queries[g], pn[sl])
        assert bad == 0, (g, worst)
        ref = parity.e2e_scores_polar(pp, rep, queries[g], pq.norms[sl], sl)
        bad, worst = parity.score_violations(s_e2e[g], ref, queries[g], pq.norms[sl])
        assert bad == 0, (g, worst)
    # stage-1 reconstruction from the oracle's codes and from the library's
    kh = _cpu(tqm.tq_dequant_mse(h, _dev(torch, pc.view(np.int32)), _dev(torch, pn)))
    bad, worst = parity.dequant_violations(kh, PL.dequant(pp, pq.codes, pn.astype(np.float64)))
    assert bad == 0, worst
    kh2 = _cpu(tqm.tq_dequant_mse(h, codes, norms))
    bad, worst = parity.dequant_violations(kh2, PL.dequant(pp, rep.reference["codes"], _cpu(norms).astype(np.float64)))
    assert bad == 0, worst


def test_polar_refused_where_unsupported(env):
    """Search, the corrected reconstruction and the value blocks take scalar
    codes only: TQ_EUNSUPPORTED, nothing launched."""
    torch, tqm = env
    _announce("polar refusals")
    h = tqm.tq_init_polar(64, 3, 1)
    keys = torch.randn((40, 64), device="cuda")
    packed = tqm.tq_quantize(h, keys)
    q = torch.randn((1, 2, 64), device="cuda")
    with pytest.raises(tqm.TqError) as e:
        tqm.tq_logits_topk(h, q, *packed, k=5)
    assert e.value.code == tqm.TQ_EUNSUPPORTED
    with pytest.raises(tqm.TqError) as e:
        tqm.tq_dequant_prod(h, *packed)
    assert e.value.code == tqm.TQ_EUNSUPPORTED
    with pytest.raises(tqm.TqError) as e:
        tqm.tq_pack_values(h, packed[0], groups=1, n=40)
    assert e.value.code == tqm.TQ_EUNSUPPORTED


@pytest.mark.timeout(300)
def test_polar_one_long_context_head_every_key(env):
    """131072 bf16 keys of one long-context head (d = 128, 3 bits): every
    angle code and sign compared, mismatches summed over all decisions and
    kept below 1e-5; scores of 4 queries against every key."""
    torch, tqm = env
    from vector_quantization_quantize_amd import workloads as wl
    w = wl.WORKLOADS["long_context"]
    _announce(f"polar long-context head: {w.n} keys d={w.d} bits={w.bits}")
    keys = wl.keys(w, 0, 0, w.n).astype(np.float64)
    queries = wl.queries(w, 0)[0]
    pp = PL.init_polar(w.d, w.bits, 0)
    h = tqm.tq_init_polar(w.d, w.bits, 0)
    codes, signs, norms, rnorms = tqm.tq_quantize(h, _dev(torch, keys.astype(np.float32), torch.bfloat16))
    scores = _cpu(tqm.tq_logits(h, _dev(torch, queries[None]), codes, signs, norms, rnorms, n=w.n))[0]
    khat = tqm.tq_dequant_mse(h, codes, norms)
    torch.cuda.synchronize()
    total = {"elements": 0, "code_mismatch": 0, "sign_mismatch": 0, "code_bad": 0, "sign_bad": 0}
    for lo in range(0, w.n, 32768):
        sl = slice(lo, lo + 32768)
        pq = PL.quantize(pp, keys[sl])
        rep = parity.compare_quantize_polar(pp, pq, _cpu(codes[sl]), _cpu(signs[sl]), _cpu(norms[sl]),
                                            _cpu(rnorms[sl]))
        assert rep.norm_bad == rep.rnorm_bad == rep.padding_bad == 0, rep
        for f in total:
            total[f] += getattr(rep, f)
        ref = parity.e2e_scores_polar(pp, rep, queries, pq.norms)
        bad, worst = parity.score_violations(scores[:, sl], ref, queries, pq.norms)
        assert bad == 0, (lo, worst)
        kref = PL.dequant(pp, rep.reference["codes"], _cpu(norms[sl]).astype(np.float64))
        bad, worst = parity.dequant_violations(_cpu(khat[sl]), kref)
        assert bad == 0, (lo, worst)
    rate = (total["code_mismatch"] + total["sign_mismatch"]) / total["elements"]
    print("polar long-context head", total, "rate", rate)
    assert total["code_bad"] == 0 and total["sign_bad"] == 0 and rate < parity.MISMATCH_RATE
