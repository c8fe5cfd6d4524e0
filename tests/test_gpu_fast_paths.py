"""Parity of the tuned d = 128 kernels (matrix-core quantize for bf16 keys,
lookup-table scorer) with the CPU oracle, on ragged tile counts, every bit
width, zero keys, exact rescaling and strided rows.  Expected values come only
from ``oracle``; rules from ``oracle.parity``."""
import os

import numpy as np
import pytest

from oracle import params as P
from oracle import tq
from tests.test_gpu_parity import _announce, _cpu, _dev, check_full

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import vector_quantization_quantize_amd as tqm
    from vector_quantization_quantize_amd import workloads as wl
    return torch, tqm, wl


def _bf16_keys(torch, rs, n, d, scale_spread=1.0):
    k = rs.standard_normal((n, d)) * np.exp(scale_spread * rs.standard_normal((n, 1)))
    return torch.tensor(k, dtype=torch.float32).bfloat16().float().numpy()


@pytest.mark.parametrize("bits,groups,n,nq", [(2, 1, 1, 1), (3, 2, 31, 4), (3, 1, 33, 5), (4, 3, 1000, 4),
                                              (5, 1, 257, 8), (3, 1, 4097, 2)])
def test_d128_bf16_fast_path(env, bits, groups, n, nq):
    torch, tqm, _ = env
    _announce(f"fast path d=128 bf16 bits={bits} groups={groups} n={n} nq={nq}")
    rs = np.random.default_rng(bits * 1000 + n)
    keys = _bf16_keys(torch, rs, groups * n, 128)
    keys[0] = 0.0
    queries = rs.standard_normal((groups, nq, 128)).astype(np.float32)
    rep = check_full(env, 128, bits, keys, queries, key_dtype="bf16", seed=bits)
    print("mismatches", rep.code_mismatch, rep.sign_mismatch, "cascade", rep.cascade_keys)


@pytest.mark.parametrize("n", [40007, 82697])
@pytest.mark.parametrize("bits", [2, 3, 4, 5])
def test_fast_paths_many_tiles_per_block(env, bits, n):
    """More tiles of 32 keys than resident blocks, the last tile ragged:
    40007 keys give the quantize kernel's blocks 2 or 3 tiles (first and
    second pass, then the last pass on either buffer), 82697 keys give 5 or 6
    (the unrolled loop, ending on either buffer); the reconstruction kernel
    loops too.  A zero key lands in a later tile.  The outputs start out as
    sentinels, so a row the kernel never writes cannot pass."""
    torch, tqm, _ = env
    from oracle import parity
    from tests.test_gpu_parity import _params
    _announce(f"fast quantize + dequant, many tiles per block: bits={bits} n={n}")
    rs = np.random.default_rng(77 + bits + n)
    keys = _bf16_keys(torch, rs, n, 128)
    keys[33333] = 0.0
    h = tqm.tq_init(128, bits, 0)
    out = tqm.empty_packed(h, n, "cuda")
    for t in out[:2]:
        t.fill_(-1)
    for t in out[2:]:
        t.fill_(float("nan"))
    out = tqm.tq_quantize(h, torch.from_numpy(keys).bfloat16().cuda(), out=out)
    pr = _params(128, bits)
    qz = tq.quantize(pr, keys.astype(np.float64))
    rep = parity.compare_quantize(pr, qz, *(_cpu(t) for t in out))
    print(rep)
    assert rep.ok(), rep
    # reconstruction of every key from the GPU's own codes and norms
    kh = _cpu(tqm.tq_dequant_mse(h, out[0], out[2]))
    idx_gpu = tq.unpack_codes(_cpu(out[0]).view(np.uint32), 128)
    bad, worst = parity.dequant_violations(kh, tq.dequant_mse(pr, idx_gpu, _cpu(out[2]).astype(np.float64)))
    assert bad == 0, (bad, worst)


def test_fast_quantize_exact_rescaling_and_strides(env):
    torch, tqm, _ = env
    _announce("fast path: power-of-two rescaling and row strides")
    rs = np.random.default_rng(11)
    keys = _bf16_keys(torch, rs, 999, 128)
    h = tqm.tq_init(128, 3, 0)
    base = torch.from_numpy(keys).bfloat16().cuda()
    a = tqm.tq_quantize(h, base)
    b = tqm.tq_quantize(h, base * 2.0 ** 40)
    c = tqm.tq_quantize(h, base * 2.0 ** -40)
    for x, y, z in zip(a[:2], b[:2], c[:2]):
        assert torch.equal(x, y) and torch.equal(x, z)
    assert torch.equal(a[3], b[3]) and torch.equal(a[3], c[3])
    assert torch.equal(a[2] * 2.0 ** 40, b[2]) and torch.equal(a[2] * 2.0 ** -40, c[2])
    # aligned row stride (fast path) and an odd one (general path) agree
    wide = torch.zeros((999, 136), dtype=torch.bfloat16, device="cuda")
    wide[:, :128] = base
    odd = torch.zeros((999, 131), dtype=torch.bfloat16, device="cuda")
    odd[:, :128] = base
    d1 = tqm.tq_quantize(h, wide[:, :128])
    d2 = tqm.tq_quantize(h, odd[:, :128])
    for x, y in zip(a, d1):
        assert torch.equal(x, y)
    # outputs that are not 16-byte aligned (norms one float into a buffer)
    # take the general path
    nbuf = torch.empty(1000, dtype=torch.float32, device="cuda")
    d3 = tqm.empty_packed(h, 999, "cuda")
    d3 = tqm.tq_quantize(h, base, out=(d3[0], d3[1], nbuf[1:], d3[3]))
    pr = P.init(128, 3, 0)
    from oracle import parity
    qz = tq.quantize(pr, keys.astype(np.float64))
    for d in (d2, d3):
        rep = parity.compare_quantize(pr, qz, *(_cpu(t) for t in d))
        assert rep.ok(), rep


def test_reference_and_fast_kernels_both_match_oracle(env):
    torch, tqm, wl = env
    _announce("reference kernels (TQ_KERNELS=ref) on the long-context generator")
    w = wl.WORKLOADS["long_context"].scaled(n=2048, groups=2)
    keys = wl.keys(w)
    queries = wl.queries(w)
    os.environ["TQ_KERNELS"] = "ref"
    try:
        check_full(env, w.d, w.bits, keys, queries, key_dtype="bf16")
    finally:
        del os.environ["TQ_KERNELS"]
    check_full(env, w.d, w.bits, keys, queries, key_dtype="bf16")


def test_logits_two_tier_key_split(env):
    """32 groups x 4 queries x 32768 keys: the scorer's grid is two blocks per
    CU on a 256-CU device, so every group's keys are cut unevenly between the
    first- and second-dispatched halves of the grid (on other CU counts the
    split is even; the results must not depend on it).  Random packed words
    (every code and sign pattern); every score is checked against the
    oracle's estimator on the same packed keys."""
    torch, tqm, _ = env
    from tests.test_gpu_parity import _params
    from oracle import parity
    d, bits, groups, nq, n = 128, 3, 32, 4, 32768
    _announce(f"logits, uneven key split: groups={groups} nq={nq} n={n} bits={bits}")
    pr = _params(d, bits)
    h = tqm.tq_init(d, bits, 0)
    rs = np.random.default_rng(4242)
    total = groups * n
    codes = rs.integers(0, 2 ** 32, size=(total, bits - 1, 4), dtype=np.uint64).astype(np.uint32)
    signs = rs.integers(0, 2 ** 32, size=(total, 4), dtype=np.uint64).astype(np.uint32)
    norms = rs.uniform(0.1, 10.0, size=total).astype(np.float32)
    rnorms = rs.uniform(0.0, 0.5, size=total).astype(np.float32)
    queries = rs.standard_normal((groups, nq, d))
    s = _cpu(tqm.tq_logits(h, _dev(torch, queries.astype(np.float32)), _dev(torch, codes.view(np.int32)),
                           _dev(torch, signs.view(np.int32)), _dev(torch, norms), _dev(torch, rnorms), n=n))
    for g in range(groups):
        sl = slice(g * n, (g + 1) * n)
        ref = tq.scores(pr, queries[g], tq.unpack_codes(codes[sl], d), tq.unpack_bits(signs[sl], d),
                        norms[sl].astype(np.float64), rnorms[sl].astype(np.float64))
        bad, worst = parity.score_violations(s[g], ref, queries[g], norms[sl])
        assert bad == 0, (g, worst)


@pytest.mark.parametrize("form", ["fused", "tiled"])
@pytest.mark.parametrize("d,bits,groups,n,key_dtype", [
    (104, 3, 1, 1000, "f32"), (128, 2, 2, 4097, "f32"), (136, 4, 1, 65, "bf16"), (168, 5, 1, 333, "f32"),
    (200, 2, 1, 3001, "f32"), (200, 5, 2, 777, "bf16"), (208, 3, 1, 2049, "f32"), (200, 3, 1, 1, "f32"),
    (128, 2, 1, 31, "bf16"), (16, 2, 1, 100, "f32"), (24, 3, 2, 77, "bf16"), (64, 4, 1, 1000, "f32"),
    (96, 5, 1, 333, "bf16")])
def test_one_kernel_quantizer(env, form, d, bits, groups, n, key_dtype):
    """Plain handles at 16 <= d <= 208 (d a multiple of 8): the one-kernel
    matrix-core quantizer, and the tiled general quantizer it replaces there
    (TQ_QUANTIZER=tiled), on ragged key counts, every bit width, a zero key
    and norms spread over many binades; codes, signs, norms, rho, scores and
    reconstructions against the oracle."""
    torch, tqm, _ = env
    _announce(f"{form} quantizer d={d} bits={bits} groups={groups} n={n} {key_dtype}")
    rs = np.random.default_rng(d * 7 + bits + n)
    keys = rs.standard_normal((groups * n, d)) * np.exp(2.0 * rs.standard_normal((groups * n, 1)))
    keys[min(5, groups * n - 1)] = 0.0
    if key_dtype == "bf16":
        keys = torch.tensor(keys, dtype=torch.float32).bfloat16().float().numpy()
    queries = rs.standard_normal((groups, 3, d)).astype(np.float32)
    old = os.environ.get("TQ_QUANTIZER")
    if form == "tiled":
        os.environ["TQ_QUANTIZER"] = "tiled"
    try:
        rep = check_full(env, d, bits, keys.astype(np.float32) if key_dtype == "f32" else keys, queries,
                         key_dtype=key_dtype, seed=bits + 1)
    finally:
        if old is None:
            os.environ.pop("TQ_QUANTIZER", None)
        else:
            os.environ["TQ_QUANTIZER"] = old
    print("mismatches", rep.code_mismatch, rep.sign_mismatch, "cascade", rep.cascade_keys)


def test_one_kernel_quantizer_strided_rows(env):
    """Rows strided by ldk > d (16-byte aligned): the one-kernel quantizer
    reads only the first d elements of each row."""
    torch, tqm, _ = env
    from oracle import parity
    from tests.test_gpu_parity import _params
    _announce("one-kernel quantizer, strided rows d=200 ldk=212")
    d, ldk, n, bits = 200, 212, 999, 3
    rs = np.random.default_rng(4242)
    keys = rs.standard_normal((n, d)).astype(np.float32)
    big = np.full((n, ldk), np.nan, dtype=np.float32)   # padding past d must never be read
    big[:, :d] = keys
    h = tqm.tq_init(d, bits, 3)
    pr = _params(d, bits, 3)
    kd = torch.from_numpy(big).cuda()
    codes, signs, norms, rnorms = tqm.tq_quantize(h, kd[:, :d])
    torch.cuda.synchronize()
    qz = tq.quantize(pr, keys.astype(np.float64))
    rep = parity.compare_quantize(pr, qz, _cpu(codes), _cpu(signs), _cpu(norms), _cpu(rnorms))
    assert rep.ok(), rep


@pytest.mark.parametrize("kind,d,bits,key_dtype", [("plain", 200, 3, "f32"), ("plain", 128, 4, "bf16"),
                                                   ("polar", 128, 3, "bf16"), ("polar", 128, 2, "f32")])
def test_new_quantizers_power_of_two_rescaling(env, kind, d, bits, key_dtype):
    """The one-kernel and polar-angle quantizers split 2^s k with 2^s n in
    [2^13, 2^14) and square and sum the key in float32, all exact under a
    power-of-two rescaling that stays in the normal range: keys times
    2^40 and 2^-40 give the same codes, signs and rho bit for bit and norms
    times exactly 2^40 and 2^-40."""
    torch, tqm, _ = env
    _announce(f"{kind} quantizer rescaling d={d} bits={bits} {key_dtype}")
    rs = np.random.default_rng(99 + d + bits)
    keys = rs.standard_normal((1500, d)).astype(np.float32)
    keys[7] = 0.0
    h = tqm.tq_init_polar(d, bits, 4) if kind == "polar" else tqm.tq_init(d, bits, 4)
    dt = torch.bfloat16 if key_dtype == "bf16" else torch.float32
    base = torch.from_numpy(keys).cuda().to(dt)
    out0 = [_cpu(t) for t in tqm.tq_quantize(h, base)]
    for e in (40, -40):
        scaled = base * (2.0 ** e)          # exact: a power of two, no overflow or subnormal
        out = [_cpu(t) for t in tqm.tq_quantize(h, scaled)]
        torch.cuda.synchronize()
        assert np.array_equal(out[0], out0[0]), "codes"
        assert np.array_equal(out[1], out0[1]), "signs"
        assert np.array_equal(out[2], out0[2] * np.float32(2.0 ** e)), "norms"
        assert np.array_equal(out[3], out0[3]), "rho"
