"""Fractional widths (tq_init_split) through the C ABI against the oracle.

The first hi rotated coordinates carry one more index bit.  Every case
prints what names it before touching the GPU; inputs are seeded, expected
values come only from ``oracle`` (``oracle.params.init_split``), and the
bars are ``oracle.parity``'s.
"""
import math
import sys

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
    return torch, tqm


def _dev(torch, a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def _cpu(t):
    return t.detach().cpu().numpy()


def _keys(rs, n, d):
    return rs.standard_normal((n, d)) * np.exp(0.5 * rs.standard_normal((n, 1)))


# (d, bits, hi, groups, n, nq): 2.5 and 3.5 bits at d = 128, ragged hi
# (one partial extra word, several words, hi = d), tiny and wide d
# d = 128 with hi = 64 also takes the matrix-core reconstruction (ragged
# tile counts: 300, 257, 4097 keys)
# bf16 keys at d = 128, hi = 64 take the matrix-core quantizer (two waves
# with the finer set; 300, 257 and 4097 keys leave ragged last tiles whose
# code rows end inside a 16-byte row)
CASES = [(128, 2, 64, 1, 300, 4, "f32"), (128, 3, 64, 2, 257, 3, "f32"), (128, 4, 64, 1, 4097, 2, "f32"),
         (40, 2, 16, 1, 77, 5, "f32"), (33, 3, 33, 2, 65, 2, "f32"), (200, 4, 100, 1, 50, 6, "f32"),
         (128, 4, 1, 1, 129, 2, "f32"), (2, 2, 1, 1, 9, 1, "f32"), (300, 2, 257, 1, 40, 3, "f32"),
         (128, 2, 64, 1, 300, 4, "bf16"), (128, 3, 64, 2, 257, 3, "bf16"), (128, 4, 64, 1, 4097, 2, "bf16"),
         (128, 3, 64, 1, 70001, 2, "bf16")]


@pytest.mark.parametrize("d,bits,hi,groups,n,nq,key_dtype", CASES)
def test_split_matches_oracle(env, d, bits, hi, groups, n, nq, key_dtype):
    """Quantize (codes, signs, norms bit for bit outside the decision
    windows), scores of the oracle's packed keys and of the library's own,
    both reconstructions, and the layout's sizes."""
    torch, tqm = env
    _announce(f"split d={d} bits={bits} hi={hi} groups={groups} n={n} nq={nq} {key_dtype}")
    pr = P.init_split(d, bits, hi, 11)
    h = tqm.tq_init_split(d, bits, hi, 11)
    w = tq.words_per_plane(d)
    assert h.layout.hi == hi and h.layout.hi_words == (hi + 31) // 32
    assert h.layout.code_bytes == 4 * ((bits - 1) * w + (hi + 31) // 32)
    rs = np.random.default_rng(d * 7 + hi)
    keys = _keys(rs, groups * n, d).astype(np.float32)
    keys[min(2, groups * n - 1)] = 0.0  # a zero key
    queries = rs.standard_normal((groups, nq, d)).astype(np.float32)
    if key_dtype == "bf16":
        kd = _dev(torch, keys).to(torch.bfloat16)
        keys = kd.float().cpu().numpy()
    else:
        kd = _dev(torch, keys)
    codes, signs, norms, rnorms = tqm.tq_quantize(h, kd)
    torch.cuda.synchronize()
    assert tuple(codes.shape) == (groups * n, (bits - 1) * w + (hi + 31) // 32)
    qz = tq.quantize(pr, keys.astype(np.float64))
    rep = parity.compare_quantize(pr, qz, _cpu(codes), _cpu(signs), _cpu(norms), _cpu(rnorms))
    assert rep.ok(), rep

    packed = tq.pack(pr, qz)
    assert np.array_equal(packed[0], _cpu(codes).view(np.uint32)) or rep.code_mismatch > 0
    pdev = (_dev(torch, packed[0].view(np.int32)), _dev(torch, packed[1].view(np.int32)),
            _dev(torch, packed[2]), _dev(torch, packed[3]))
    qd = _dev(torch, queries)
    s_dec = _cpu(tqm.tq_logits(h, qd, *pdev, n=n))
    s_e2e = _cpu(tqm.tq_logits(h, qd, codes, signs, norms, rnorms, n=n))
    for g in range(groups):
        sl = slice(g * n, (g + 1) * n)
        ref = tq.scores(pr, queries[g], qz.idx[sl], qz.beta[sl], packed[2][sl].astype(np.float64),
                        packed[3][sl].astype(np.float64))
        bad, worst = parity.score_violations(s_dec[g], ref, queries[g], packed[2][sl])
        assert bad == 0, (g, worst)
        ref = parity.e2e_scores(pr, rep, queries[g], qz.norms[sl], sl)
        bad, worst = parity.score_violations(s_e2e[g], ref, queries[g], qz.norms[sl])
        assert bad == 0, (g, worst)

    kh = _cpu(tqm.tq_dequant_mse(h, pdev[0], pdev[2]))
    bad, worst = parity.dequant_violations(kh, tq.dequant_mse(pr, qz.idx, packed[2].astype(np.float64)))
    assert bad == 0, worst
    kt = _cpu(tqm.tq_dequant_prod(h, *pdev))
    bad, worst = parity.dequant_violations(kt, tq.dequant_prod(pr, qz.idx, qz.beta, packed[2].astype(np.float64),
                                                               packed[3].astype(np.float64)))
    assert bad == 0, worst


@pytest.mark.parametrize("d,bits,hi,n,nq,k", [(128, 3, 64, 5000, 8, 10), (40, 2, 20, 700, 3, 64)])
def test_split_topk_matches_oracle(env, d, bits, hi, n, nq, k):
    """Search with fractional widths: the k best of the oracle's packed keys
    per query, checked by the search parity rules (unique best scores,
    ties only within the score bar)."""
    torch, tqm = env
    _announce(f"split top-k d={d} bits={bits} hi={hi} n={n} nq={nq} k={k}")
    pr = P.init_split(d, bits, hi, 4)
    h = tqm.tq_init_split(d, bits, hi, 4)
    rs = np.random.default_rng(n + hi)
    keys = _keys(rs, n, d)
    queries = rs.standard_normal((1, nq, d)).astype(np.float32)
    qz = tq.quantize(pr, keys)
    packed = tq.pack(pr, qz)
    pdev = (_dev(torch, packed[0].view(np.int32)), _dev(torch, packed[1].view(np.int32)),
            _dev(torch, packed[2]), _dev(torch, packed[3]))
    idx, sc = tqm.tq_logits_topk(h, _dev(torch, queries), *pdev, k)
    torch.cuda.synchronize()
    ref = tq.scores(pr, queries[0], qz.idx, qz.beta, packed[2].astype(np.float64), packed[3].astype(np.float64))
    rep = parity.compare_topk(_cpu(idx)[0], _cpu(sc)[0], ref, queries[0], packed[2], k)
    assert rep.ok(), rep.bad[:3]


def test_split_keys_in_attention(env):
    """Decode attention with a fractional-width key handle and a plain value
    handle, against the oracle's attention of the same packed cache."""
    torch, tqm = env
    d, groups, nq, n = 128, 2, 4, 600
    _announce(f"split-key attention d={d} groups={groups} nq={nq} n={n}")
    prk, prv = P.init_split(d, 3, 64, 0), P.init(d, 3, 1)
    hk, hv = tqm.tq_init_split(d, 3, 64, 0), tqm.tq_init(d, 3, 1)
    rs = np.random.default_rng(5)
    keys, vals = _keys(rs, groups * n, d), _keys(rs, groups * n, d)
    queries = rs.standard_normal((groups, nq, d)).astype(np.float32)
    kz, vz = tq.quantize(prk, keys), tq.quantize(prv, vals)
    kc, ks, kn, kr = tq.pack(prk, kz)
    vc = tq.pack_codes(vz.idx, prv.code_bits)
    vn = vz.norms.astype(np.float32)
    blocks = tqm.tq_pack_values(hv, _dev(torch, vc.view(np.int32)), groups=groups, n=n)
    scale = 1.0 / math.sqrt(d)
    out, lse = tqm.tq_attention(hk, hv, _dev(torch, queries), _dev(torch, kc.view(np.int32)),
                                _dev(torch, ks.view(np.int32)), _dev(torch, kn), _dev(torch, kr), blocks,
                                _dev(torch, vn), scale=scale, n=n)
    torch.cuda.synchronize()
    out, lse = _cpu(out), _cpu(lse)
    for g in range(groups):
        sl = slice(g * n, (g + 1) * n)
        o, l = tq.attention(prk, prv, queries[g], kz.idx[sl], kz.beta[sl], kn[sl].astype(np.float64),
                            kr[sl].astype(np.float64), vz.idx[sl], vn[sl].astype(np.float64), scale)
        vh = tq.dequant_mse(prv, vz.idx[sl], vn[sl].astype(np.float64))
        qn = np.sqrt((queries[g].astype(np.float64) ** 2).sum(axis=1))
        delta = scale * 1e-3 * qn * kn[sl].max()
        tol_o = np.expm1(2 * delta)[:, None] * np.abs(vh).max(axis=0)[None, :] + 2e-5 * np.sqrt((vh * vh).sum(1)).max()
        assert np.all(np.abs(out[g] - o) <= tol_o)
        assert np.all(np.abs(lse[g] - l) <= delta + 1e-5 * np.maximum(1.0, np.abs(l)))


def test_split_rejections(env):
    """Stored values use one width: a fractional-width value handle is
    refused by the value packer and by attention."""
    torch, tqm = env
    _announce("split rejections")
    hs, hk = tqm.tq_init_split(128, 3, 64, 0), tqm.tq_init(128, 3, 0)
    codes = torch.zeros((64, hs.code_shape[0]), dtype=torch.int32, device="cuda")
    with pytest.raises(tqm.TqError) as e:
        tqm.tq_pack_values(hs, codes, groups=1, n=64)
    assert e.value.code == tqm.TQ_EUNSUPPORTED
    dummy = torch.zeros(4096, dtype=torch.int32, device="cuda")
    with pytest.raises(tqm.TqError) as e:
        tqm.tq_attention(hk, hs, torch.ones((1, 4, 128), device="cuda"), dummy, dummy, dummy.float(), dummy.float(),
                         dummy, dummy.float(), n=32)
    assert e.value.code == tqm.TQ_EUNSUPPORTED


def test_split_hi_zero_is_the_plain_handle(env):
    """hi = 0 builds exactly tq_init's parameters and packed format: same
    parameter hash, layout and bit-identical quantizer output."""
    torch, tqm = env
    _announce("split hi=0 equals plain")
    a, b = tqm.tq_init_split(128, 3, 0, 9), tqm.tq_init(128, 3, 9)
    assert tqm.tq_params_hash(a) == tqm.tq_params_hash(b)
    assert a.code_shape == b.code_shape == (2, 4) and a.layout.code_bytes == b.layout.code_bytes
    keys = _dev(torch, _keys(np.random.default_rng(3), 500, 128), torch.bfloat16)
    pa, pb = tqm.tq_quantize(a, keys), tqm.tq_quantize(b, keys)
    torch.cuda.synchronize()
    for x, y in zip(pa, pb):
        assert torch.equal(x, y)
