"""tq_logits_noalloc (the allocation-free variant of tq_logits) against
tq_logits through the C ABI: identical scores on two calls in a row, the
second with a smaller input, on every scorer path that takes a workspace
(matrix-core scorer, general scorer, tiled scorer for d > 256) and on the
lookup-table path; a request larger than the static scratch is refused
before anything is launched."""
import sys

import numpy as np
import pytest

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


# (d, bits, groups, nq, n) first call, then a smaller (groups, nq, n)
CASES = [
    (128, 3, (2, 20, 3000), (1, 17, 1000)),     # matrix-core scorer (nq >= 16)
    (200, 4, (3, 4, 2000), (2, 3, 700)),        # general scorer
    (300, 3, (1, 130, 600), (1, 40, 257)),      # tiled scorer (d > 256): float16 query rows in the scratch
    (128, 4, (8, 4, 4096), (2, 4, 100)),        # lookup-table scorer (no workspace use)
]


@pytest.mark.parametrize("d,bits,first,second", CASES)
def test_noalloc_matches_tq_logits(env, d, bits, first, second):
    torch, tqm = env
    h = tqm.tq_init(d, bits, 3)
    rs = np.random.default_rng(d + bits)
    for groups, nq, n in (first, second):
        _announce(f"tq_logits_noalloc d={d} bits={bits} groups={groups} nq={nq} n={n}")
        keys = torch.from_numpy(rs.standard_normal((groups * n, d)).astype(np.float32)).cuda()
        q = torch.from_numpy(rs.standard_normal((groups, nq, d)).astype(np.float32)).cuda()
        packed = tqm.tq_quantize(h, keys)
        ref = tqm.tq_logits(h, q, *packed, n=n)
        out = torch.full((groups, nq, n), float("nan"), dtype=torch.float32, device="cuda")
        got = tqm.tq_logits_noalloc(h, q, *packed, n=n, scores=out)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert torch.equal(got, ref), (d, bits, groups, nq, n)


def test_noalloc_refuses_requests_beyond_the_scratch(env):
    torch, tqm = env
    _announce("tq_logits_noalloc size limit")
    h = tqm.tq_init(128, 3, 0)
    cap = tqm.tq_noalloc_scratch_bytes()
    assert cap == 16 << 20
    per_row = tqm.tq_logits_workspace_size(h, 1, 256) // 256
    rows = cap // per_row + 256
    assert tqm.tq_logits_workspace_size(h, 1, rows) > cap
    keys = torch.zeros((64, 128), dtype=torch.float32, device="cuda")
    packed = tqm.tq_quantize(h, keys)
    q = torch.zeros((1, rows, 128), dtype=torch.float32, device="cuda")
    scores = torch.empty((1, rows, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(tqm.TqError) as exc:
        tqm.tq_logits_noalloc(h, q, *packed, n=64, scores=scores)
    assert exc.value.code == tqm.TQ_ESCRATCH
