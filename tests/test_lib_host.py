"""CPU checks of libtq: it loads, exports every declared symbol, builds the
same parameters as the oracle, and rejects bad arguments without a GPU."""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import params as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tq.h")


@pytest.fixture(scope="module")
def tqm():
    import vector_quantization_quantize_amd as tqm
    return tqm


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"TQ_API\s+[\w\s\*]+?\b(tq_\w+)\s*\(", text)))


def test_header_declares_and_library_exports_everything(tqm):
    names = _declared()
    assert len(names) == len(tqm.EXPORTS) and sorted(tqm.EXPORTS) == names
    lib = ctypes.CDLL(tqm.LIB_PATH)
    for name in names:
        assert hasattr(lib, name), name


def _ulps(a, b):
    a = np.asarray(a, dtype=np.float32).view(np.int32).astype(np.int64)
    b = np.asarray(b, dtype=np.float32).view(np.int32).astype(np.int64)
    return np.abs(a - b)


@pytest.mark.parametrize("d,bits,seed", [(2, 2, 0), (4, 3, 1), (33, 5, 2), (128, 3, 0), (128, 4, 0),
                                         (200, 2, 0), (200, 4, 0)])
def test_host_params_match_oracle(tqm, d, bits, seed):
    """The C++ builder (Householder QR, Gauss-Legendre Lloyd-Max) and the
    oracle (LAPACK QR, incomplete-beta Lloyd-Max) agree to <= 1 float32 ulp."""
    pi, g, c, t = tqm.tq_host_params(d, bits, seed)
    pr = P.init(d, bits, seed)
    assert _ulps(pi, pr.pi).max() <= 1
    assert (_ulps(pi, pr.pi) > 0).mean() < 1e-4
    assert np.array_equal(g, pr.g.astype(np.float32))
    assert np.array_equal(g.astype(np.float16).astype(np.float32), g)  # float16-exact G
    assert _ulps(c, pr.centroids).max() <= 1
    assert _ulps(t, pr.thresholds).max() <= 1


@pytest.mark.parametrize("d", [2, 4, 64, 128, 1024])
def test_hadamard_rotation_matches_oracle(tqm, d):
    """The C++ and oracle randomized Hadamard rotations agree bit for bit
    (both round +-1/sqrt(d) once to float32 and draw the same signs)."""
    pi = tqm.tq_hadamard_rotation(d, 7)
    assert np.array_equal(pi.astype(np.float64), P.hadamard_rotation(d, 7))


def test_hadamard_rejects_other_d(tqm):
    lib = tqm._lib()
    out = ctypes.c_void_p()
    buf = np.empty(100 * 100, dtype=np.float32)
    for d in (1, 3, 100, 8192):
        assert lib.tq_init_hadamard(d, 3, 0, ctypes.byref(out)) == tqm.TQ_EINVAL
        assert lib.tq_hadamard_rotation(d, 0, buf.ctypes.data) == tqm.TQ_EINVAL


def test_host_params_d1536(tqm):
    pi, g, c, t = tqm.tq_host_params(1536, 4, 0)
    pr = P.init(1536, 4, 0)
    assert _ulps(pi, pr.pi).max() <= 1
    assert (_ulps(pi, pr.pi) > 0).sum() <= 8
    assert np.array_equal(c, pr.centroids.astype(np.float32))


def test_bad_arguments_are_rejected(tqm):
    lib = tqm._lib()
    out = ctypes.c_void_p()
    for d, bits in [(1, 3), (4097, 3), (128, 1), (128, 6)]:
        assert lib.tq_init(d, bits, 0, ctypes.byref(out)) == tqm.TQ_EINVAL
    assert lib.tq_init(128, 3, 0, None) == tqm.TQ_EINVAL
    # fractional widths: hi in [0, d], bits <= 4 when hi > 0
    for d, bits, hi in [(128, 3, -1), (128, 3, 129), (128, 5, 1), (1, 3, 0), (40, 1, 3)]:
        assert lib.tq_init_split(d, bits, hi, 0, ctypes.byref(out)) == tqm.TQ_EINVAL
    assert lib.tq_init_split(128, 3, 64, 0, None) == tqm.TQ_EINVAL
    assert lib.tq_host_params(0, 3, 0, None, None, None, None) == tqm.TQ_EINVAL
    assert lib.tq_quantize(None, None, 0, 1, 128, None, None, None, None, None) == tqm.TQ_EINVAL
    assert lib.tq_logits(None, None, 1, 1, None, None, None, None, 1, None, None, 0, None) == tqm.TQ_EINVAL
    assert lib.tq_dequant_mse(None, None, None, 1, None, None) == tqm.TQ_EINVAL
    assert lib.tq_logits_topk(None, None, 1, 1, None, None, None, None, 1, 10, None, None, None, 0,
                              None) == tqm.TQ_EINVAL
    assert lib.tq_logits_topk_workspace_size(None, 1, 1, 1, 10) == 0
    assert lib.tq_pack_values(None, None, 1, 1, None, None) == tqm.TQ_EINVAL
    assert lib.tq_dequant_prod(None, None, None, None, None, 1, None, None) == tqm.TQ_EINVAL
    assert lib.tq_dense_logits(None, 1, 1, None, 0, 1, 128, 128, None, None) == tqm.TQ_EINVAL
    assert lib.tq_dense_logits(None, 1, 1, None, 2, 1, 128, 128, None, None) == tqm.TQ_EINVAL
    assert lib.tq_attention_workspace_size(None, None, 1, 1, 1) == 0
    assert lib.tq_attention(None, None, None, 1, 1, None, None, None, None, None, None, 1, 0.1, None, None, None,
                            0, None) == tqm.TQ_EINVAL
    assert lib.tq_destroy(None) == tqm.TQ_OK
    assert lib.tq_params_hash(None) == 0
    assert lib.tq_logits_workspace_size(None, 1, 1) == 0
    assert lib.tq_strerror(tqm.TQ_EINVAL) == b"invalid argument"
    assert lib.tq_strerror(12345) == b"unknown error"


def test_host_params_null_outputs_skip(tqm):
    lib = tqm._lib()
    c = np.empty(4, dtype=np.float32)
    assert lib.tq_host_params(16, 3, 0, None, None, c.ctypes.data, None) == 0
    assert np.array_equal(c, P.init(16, 3, 0).centroids.astype(np.float32))


@pytest.mark.parametrize("d,bits", [(2, 2), (16, 3), (128, 3), (128, 4), (1024, 2), (4096, 5)])
def test_polar_codebooks_match_oracle(tqm, d, bits):
    """Polar angle codebooks: the C++ builder (Lloyd-Max in theta = 2 psi -
    pi/2 by Gauss-Legendre panels) and the oracle (Lloyd-Max in phi = psi -
    pi/4 with incomplete-beta masses and adaptive quadrature moments) agree
    to <= 1 float32 ulp on every level; thresholds are the same midpoints."""
    from oracle import polar as PL
    L = 1 << (bits - 1)
    nl = d.bit_length() - 1
    levels = list(range(1, nl + 1)) if nl <= 4 else [1, 2, 3, nl - 1, nl]
    for lvl in levels:
        c, t = tqm.tq_polar_codebook(d, bits, lvl)
        if lvl == 1:
            c_or = ((np.arange(L) + 0.5) * PL.TWO_PI / L).astype(np.float32)
            t_or = (np.arange(1, L) * PL.TWO_PI / L).astype(np.float32)
        else:
            c_or = PL.level_codebook_fp64(1 << (lvl - 1), L).astype(np.float32)
            t_or = P.thresholds_from_centroids(c_or).astype(np.float32)
        assert _ulps(c, c_or).max() <= 1, (lvl, c, c_or)
        assert _ulps(t, t_or).max() <= 1, (lvl, t, t_or)


def test_polar_init_rejects_bad_arguments(tqm):
    """d not a power of two, or bits out of range: TQ_EINVAL without a GPU
    call; the host codebook refuses a level past log2 d."""
    out = ctypes.c_void_p()
    lib = tqm._lib()
    assert lib.tq_init_polar(200, 3, 0, ctypes.byref(out)) == tqm.TQ_EINVAL
    assert lib.tq_init_polar(1, 3, 0, ctypes.byref(out)) == tqm.TQ_EINVAL
    assert lib.tq_polar_codebook(128, 3, 8, None, None) == tqm.TQ_EINVAL
    assert lib.tq_polar_codebook(128, 6, 1, None, None) == tqm.TQ_EINVAL
