"""Search entry point (tq_logits_topk): the k best keys per query against the
oracle's top-k of its own scores on the same packed keys (rule in
``oracle.parity.compare_topk``), including many score chunks, k past n,
partial query quads, several groups and equal scores; recall against exact
inner products on the search workload's generator.  Both forms: chunked
(score chunks, then merge; forced by TQ_TOPK_CHUNK) and fused (the
matrix-core scorer keeps per-block lists; taken for 16 or more queries when
no chunk size is forced: register form for d <= 256, tiled form above).  Expected values come only from
``oracle``."""
import os

import numpy as np
import pytest

from oracle import parity
from oracle import tq
from tests.test_gpu_parity import _announce, _cpu, _dev, _packed_to_dev, _params

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import vector_quantization_quantize_amd as tqm
    from vector_quantization_quantize_amd import workloads as wl
    return torch, tqm, wl


def _check_topk(env, d, bits, keys, queries, k, chunk=None):
    """Quantize on the oracle, score and select on the GPU from the oracle's
    packed keys; returns (gpu indices, oracle top-k indices) per group."""
    torch, tqm, _ = env
    pr = _params(d, bits)
    h = tqm.tq_init(d, bits, 0)
    groups, nq, _ = queries.shape
    n = keys.shape[0] // groups
    qz = tq.quantize(pr, keys.astype(np.float64))
    packed = tq.pack(pr, qz)
    pdev = _packed_to_dev(torch, packed)
    old = os.environ.get("TQ_TOPK_CHUNK")
    if chunk is not None:
        os.environ["TQ_TOPK_CHUNK"] = str(chunk)
    try:
        idx, sc = tqm.tq_logits_topk(h, _dev(torch, queries.astype(np.float32)), *pdev, k=k, n=n)
        torch.cuda.synchronize()
    finally:
        if chunk is not None:
            if old is None:
                del os.environ["TQ_TOPK_CHUNK"]
            else:
                os.environ["TQ_TOPK_CHUNK"] = old
    idx, sc = _cpu(idx), _cpu(sc)
    found, ref = [], []
    for g in range(groups):
        sl = slice(g * n, (g + 1) * n)
        s_ref = tq.scores(pr, queries[g], qz.idx[sl], qz.beta[sl], packed[2][sl].astype(np.float64),
                          packed[3][sl].astype(np.float64))
        kk = min(k, n)
        rep = parity.compare_topk(idx[g][:, :kk], sc[g][:, :kk], s_ref, queries[g], packed[2][sl], k)
        assert rep.ok(), (g, rep.bad[:5])
        if k > n:  # entries past n are empty
            assert np.all(idx[g][:, n:] == -1) and np.all(np.isneginf(sc[g][:, n:]))
        found.append(idx[g][:, :kk])
        ref.append(tq.topk(s_ref, kk)[0])
        print("group", g, "near-k swaps", rep.swapped)
    return found, ref


@pytest.mark.parametrize("d,bits,groups,nq,n,k,chunk", [
    (128, 3, 1, 4, 3000, 10, 256),     # table scorer, 12 chunks, ragged last
    (128, 2, 2, 5, 1000, 16, None),    # two groups, partial query quad, one chunk
    (100, 4, 1, 1, 777, 1, 64),        # top-1, d < 128 on the table scorer
    (200, 2, 1, 6, 2050, 10, 512),     # general scorer (d = 200), several chunks
    (64, 5, 3, 2, 7, 10, None),        # k > n
    (256, 3, 1, 3, 640, 64, 128),      # k at its maximum, general scorer
])
def test_topk_matches_oracle(env, d, bits, groups, nq, n, k, chunk):
    _announce(f"topk d={d} bits={bits} groups={groups} nq={nq} n={n} k={k} chunk={chunk}")
    rs = np.random.default_rng(d + bits + n)
    keys = rs.standard_normal((groups * n, d))
    queries = rs.standard_normal((groups, nq, d)).astype(np.float32)
    _check_topk(env, d, bits, keys, queries, k, chunk)


@pytest.mark.parametrize("d,bits,groups,nq,n,k", [
    (128, 3, 1, 16, 3000, 10),    # fewest queries of the fused form
    (200, 2, 1, 130, 2050, 10),   # one index bit (sign form), two query tiles, ragged key tile
    (256, 5, 2, 33, 700, 64),     # k at its maximum, four index bits, two groups
    (33, 4, 1, 20, 7, 10),        # k > n, one partial key tile
    (100, 2, 3, 17, 300, 1),      # top-1, sign form, three groups
    (64, 2, 1, 40, 40000, 5),     # many blocks per query tile
    (48, 4, 1, 300, 5000, 32),    # three query tiles, three index bits
    (1536, 4, 1, 40, 3000, 10),   # tiled form (d > 256), three index bits
    (300, 2, 2, 20, 1000, 16),    # tiled form, sign form, two groups
    (257, 3, 1, 130, 700, 64),    # tiled form at its smallest d, k at its maximum, two query tiles
])
def test_topk_fused_matches_oracle(env, d, bits, groups, nq, n, k):
    _announce(f"topk fused d={d} bits={bits} groups={groups} nq={nq} n={n} k={k}")
    rs = np.random.default_rng(d * 3 + bits + n + k)
    keys = rs.standard_normal((groups * n, d))
    queries = rs.standard_normal((groups, nq, d)).astype(np.float32)
    _check_topk(env, d, bits, keys, queries, k)


@pytest.mark.parametrize("nq,chunk", [(4, 128), (20, None)])
def test_topk_equal_scores_in_index_order(env, nq, chunk):
    """Every key appears three times: equal packed keys get equal scores, and
    the three copies must come out in ascending index order (chunked form,
    and the fused form, where copies fall in different key tiles)."""
    _announce(f"topk equal scores nq={nq} chunk={chunk}")
    rs = np.random.default_rng(9)
    base = rs.standard_normal((200, 128))
    keys = np.concatenate([base, base, base])
    queries = rs.standard_normal((1, nq, 128)).astype(np.float32)
    found, _ = _check_topk(env, 128, 3, keys, queries, 12, chunk=chunk)
    for row in found[0]:
        copies = {}
        for pos, i in enumerate(row.tolist()):
            copies.setdefault(i % 200, []).append(i)
        for lst in copies.values():
            assert lst == sorted(lst)


@pytest.mark.parametrize("name,chunk,n", [("search_b2", 8192, 60000), ("search_b4", 8192, 60000),
                                          ("search_b2", None, 60000), ("search_b4", None, 60000),
                                          ("cone", None, 20000)])
def test_topk_search_recall(env, name, chunk, n):
    """The search workloads' generators (d = 200 anisotropic; d = 1536 cone,
    which takes the tiled scorer) at n keys and 32 queries: parity of the
    top-10 with the oracle, and recall against exact inner products of the
    unquantized vectors equal to the oracle's own (the sets may differ only
    at the 10th score)."""
    torch, tqm, wl = env
    w = wl.WORKLOADS[name].scaled(n=n, nq=32)
    _announce(f"topk recall {w.name} n={w.n} nq={w.nq} bits={w.bits} chunk={chunk}")
    keys = wl.keys(w)
    queries = wl.queries(w)
    found, ref = _check_topk(env, w.d, w.bits, keys, queries, 10, chunk=chunk)
    exact = tq.exact_inner_products(queries[0], keys)
    exact_idx, _ = tq.topk(exact, 10)
    r_gpu = tq.recall_at_k(found[0], exact_idx)
    r_ref = tq.recall_at_k(ref[0], exact_idx)
    r1_gpu = tq.recall_1_at_k(found[0], exact_idx[:, 0])
    r1_ref = tq.recall_1_at_k(ref[0], exact_idx[:, 0])
    print(f"{w.name}: recall@10 gpu {r_gpu:.3f} oracle {r_ref:.3f}; Recall@1@10 gpu {r1_gpu:.3f} oracle {r1_ref:.3f}")
    assert abs(r_gpu - r_ref) <= 0.05 and abs(r1_gpu - r1_ref) <= 0.1


@pytest.mark.parametrize("d,bits,groups,nq,n", [
    (128, 3, 1, 16, 1000),   # fewest queries that take the matrix-core scorer
    (200, 2, 1, 130, 777),   # two query tiles, the second nearly empty; ragged key tile
    (256, 5, 2, 33, 65),     # d at its maximum, two groups
    (33, 4, 1, 20, 500),     # d not a multiple of 16
    (2, 2, 1, 16, 40),       # smallest d
    (100, 3, 3, 17, 300),
    (300, 2, 1, 20, 300),    # tiled form (d > 256): sign form, ragged key tile
    (1536, 4, 1, 130, 200),  # tiled form, two query tiles
    (257, 5, 2, 17, 150),    # tiled form at its smallest d, four index bits, two groups
    (1024, 3, 1, 16, 129),   # tiled form, one float16 piece per level
])
def test_matrix_core_scorer_every_score(env, d, bits, groups, nq, n):
    """Many queries per group go to the matrix-core scorer: every score of
    the oracle's packed keys against the oracle's estimator."""
    torch, tqm, _ = env
    _announce(f"matrix-core scorer d={d} bits={bits} groups={groups} nq={nq} n={n}")
    pr = _params(d, bits)
    h = tqm.tq_init(d, bits, 0)
    rs = np.random.default_rng(d * 7 + nq + n)
    keys = rs.standard_normal((groups * n, d)) * np.exp(0.5 * rs.standard_normal((groups * n, 1)))
    queries = rs.standard_normal((groups, nq, d)).astype(np.float32) * 3.0
    qz = tq.quantize(pr, keys)
    packed = tq.pack(pr, qz)
    pdev = _packed_to_dev(torch, packed)
    s = _cpu(tqm.tq_logits(h, _dev(torch, queries), *pdev, n=n))
    worst = 0.0
    for g in range(groups):
        sl = slice(g * n, (g + 1) * n)
        ref = tq.scores(pr, queries[g], qz.idx[sl], qz.beta[sl], packed[2][sl].astype(np.float64),
                        packed[3][sl].astype(np.float64))
        bad, ratio = parity.score_violations(s[g], ref, queries[g], packed[2][sl])
        assert bad == 0, (g, ratio)
        worst = max(worst, ratio)
    print(f"worst |error| / tolerance {worst:.3f}")
