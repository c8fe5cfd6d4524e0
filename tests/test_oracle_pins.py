"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test names the part of the oracle it pins and the source of the
expected value: a worked example printed on the pages, a published table, a
closed form, an invariant or brute force.  A plausible slip in the oracle (a
dropped term, a wrong sign, a transposed operand, a wrong index) fails at
least one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
from scipy import integrate, stats

from oracle import params as P
from oracle import rng
from oracle import tq

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# generator
# ---------------------------------------------------------------------------

def test_splitmix64_reference_outputs():
    """fmix64 + counter match the published SplitMix64 outputs for state 0."""
    g = _golden("splitmix64_seed0.json")
    out = rng.splitmix64_sequence(g["state"], len(g["first_outputs_hex"]))
    assert [int(x) for x in out] == [int(h, 16) for h in g["first_outputs_hex"]]


def test_normals_are_standard_normal():
    """Box-Muller pairs: both the cosine and the sine halves are N(0, 1)."""
    x = rng.normals(7, 0, 200000)
    for half in (x[0::2], x[1::2]):
        assert stats.kstest(half, "norm").pvalue > 1e-3
    # the two members of a pair are uncorrelated
    assert abs(np.corrcoef(x[0::2], x[1::2])[0, 1]) < 0.02


def test_normals_counter_based_prefix_and_streams():
    a = rng.normals(3, 1, 1001)
    assert np.array_equal(a[:500], rng.normals(3, 1, 500))
    b = rng.normals(3, 0, 1001)
    assert not np.allclose(a, b)
    assert abs(np.corrcoef(a, b)[0, 1]) < 0.1


# ---------------------------------------------------------------------------
# rotation (Haar)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d", [4, 33, 128])
def test_rotation_is_orthogonal(d):
    """P1: Pi Pi^T = I and ||Pi x|| = ||x|| (float32-rounded Pi)."""
    pr = P.init(d, 3, 11)
    assert np.max(np.abs(pr.pi @ pr.pi.T - np.eye(d))) <= 1e-6
    x = np.random.default_rng(0).standard_normal((16, d))
    ratio = np.linalg.norm(x @ pr.pi.T, axis=1) / np.linalg.norm(x, axis=1)
    assert np.max(np.abs(ratio - 1.0)) <= 1e-6


def test_pages_4d_rotation_example():
    """P2: the pages' 4-D example, rotating a one-axis vector to [5,5,5,5]."""
    g = _golden("polarquant_4d_example.json")
    q = np.array(g["rotation"])
    x = np.array(g["input"])
    assert np.max(np.abs(q @ q.T - np.eye(4))) == 0.0
    pr = P.explicit(4, 3, q, np.eye(4))
    norms, u = tq.normalize(x[None, :])
    z = tq.rotate(pr, u)
    assert norms[0] == 10.0
    assert np.array_equal(norms[0] * z[0], np.array(g["expected"]))


def test_haar_spreads_one_axis_fourth_moment():
    """P3: sum_j (Pi e1)_j^4 averages 3/(d+2) for a uniform unit vector."""
    d = 16
    vals = []
    for seed in range(300):
        col = P.haar_rotation(d, seed)[:, 0]
        vals.append(np.sum(col ** 4))
    vals = np.array(vals)
    expect = 3.0 / (d + 2)
    assert abs(vals.mean() - expect) < 4 * vals.std() / math.sqrt(len(vals))


def test_haar_sign_fix_centres_diagonal():
    """Without the sign fix a QR factor has a biased diagonal; Haar has mean 0."""
    d = 8
    diag = np.array([np.diag(P.haar_rotation(d, s)) for s in range(400)])
    sd = diag.std(axis=0) / math.sqrt(diag.shape[0])
    assert np.all(np.abs(diag.mean(axis=0)) < 4.5 * sd)


def test_rotated_coordinate_marginal_matches_beta_law():
    """P4: pooled coordinates of Pi u follow f_d (its CDF is a beta CDF)."""
    d = 12
    # one coordinate of Pi e_1 per seed: independent draws of f_d
    z = np.array([P.haar_rotation(d, seed)[seed % d, 0] for seed in range(3000)])
    assert stats.kstest(z, lambda t: P.sphere_marginal_cdf(t, d)).pvalue > 1e-3
    # and not merely the large-d normal limit it resembles
    assert stats.kstest(z * math.sqrt(d), "norm").pvalue < stats.kstest(
        z, lambda t: P.sphere_marginal_cdf(t, d)).pvalue


def test_projection_is_iid_standard_normal():
    pr = P.init(64, 3, 2)
    g = pr.g.ravel()
    assert stats.kstest(g, "norm").pvalue > 1e-3
    assert not np.allclose(np.abs(pr.g[:4, :4]), np.abs(pr.pi[:4, :4]) * 8)


# ---------------------------------------------------------------------------
# codebook (Lloyd-Max)
# ---------------------------------------------------------------------------

def _gauss_mse(c):
    t = np.concatenate(([-np.inf], 0.5 * (c[:-1] + c[1:]), [np.inf]))
    m0 = stats.norm.cdf(t[1:]) - stats.norm.cdf(t[:-1])
    m1 = stats.norm.pdf(t[:-1]) - stats.norm.pdf(t[1:])
    return 1.0 - np.sum(c * (2 * m1 - c * m0))


@pytest.mark.parametrize("levels", [2, 4, 8, 16])
def test_lloyd_max_reproduces_max_1960(levels):
    """P5: the Lloyd-Max routine on N(0,1) gives Max's published quantizers."""
    g = _golden("max1960_gaussian.json")
    row = g["levels"][str(levels)]
    tol = g["tolerance"]
    c, _ = P.gaussian_codebook_fp64(levels)
    pos = c[levels // 2:]
    assert np.max(np.abs(pos - np.array(row["outputs"]))) <= tol * max(1.0, pos.max())
    t = 0.5 * (c[:-1] + c[1:])
    tpos = t[levels // 2:]
    if row["thresholds"]:
        assert np.max(np.abs(tpos - np.array(row["thresholds"]))) <= tol * max(1.0, tpos.max())
    assert abs(_gauss_mse(c) - row["mse"]) <= 2e-4 * max(1.0, row["mse"] * 10)


@pytest.mark.parametrize("levels", [2, 4, 8])
def test_codebook_d3_is_uniform_quantizer(levels):
    """P5: at d = 3 the marginal is uniform on [-1,1]; Lloyd-Max is uniform."""
    c, _ = P.sphere_codebook_fp64(3, levels)
    expect = -1.0 + (2.0 * np.arange(levels) + 1.0) / levels
    assert np.max(np.abs(c - expect)) < 1e-12
    assert abs(3 * P.codebook_mse(c, 3) - 4.0 ** -int(math.log2(levels))) < 1e-12


def test_codebook_large_d_tends_to_gaussian():
    """sqrt(d) c(d) tends to the N(0,1) quantizer as d grows."""
    cg, _ = P.gaussian_codebook_fp64(8)
    c, _ = P.sphere_codebook_fp64(4096, 8)
    assert np.max(np.abs(np.sqrt(4096) * c - cg)) < 2e-3


@pytest.mark.parametrize("d,levels", [(5, 4), (128, 4), (200, 8), (1536, 8)])
def test_codebook_fixed_point_by_quadrature(d, levels):
    """P6: each level is the conditional mean of its cell (independent quad)."""
    c, _ = P.sphere_codebook_fp64(d, levels)
    t = np.concatenate(([-1.0], 0.5 * (c[:-1] + c[1:]), [1.0]))
    s = 1.0 / math.sqrt(d)
    for i in range(levels):
        a, b = max(t[i], -40 * s), min(t[i + 1], 40 * s)
        m0 = integrate.quad(lambda z: P.sphere_marginal_pdf(z, d), a, b, epsabs=0, epsrel=1e-12, limit=200)[0]
        m1 = integrate.quad(lambda z: z * P.sphere_marginal_pdf(z, d), a, b, epsabs=0, epsrel=1e-12, limit=200)[0]
        assert abs(m1 / m0 - c[i]) <= 1e-9 * s
    assert np.array_equal(c, -c[::-1])


def test_marginal_pdf_normalised_and_moment_formula():
    for d in (2, 3, 9, 128):
        tot = integrate.quad(lambda z: P.sphere_marginal_pdf(z, d), -1, 1, limit=200)[0]
        assert abs(tot - 1.0) < 1e-8
        m = integrate.quad(lambda z: z * P.sphere_marginal_pdf(z, d), 0.1, 0.4, limit=200)[0]
        assert abs(m - P.sphere_marginal_moment(0.1, 0.4, d)) < 1e-12
        var = integrate.quad(lambda z: z * z * P.sphere_marginal_pdf(z, d), -1, 1, limit=200)[0]
        assert abs(var - 1.0 / d) < 1e-9


def test_mse_falls_about_4x_per_bit_and_within_27x_of_bound():
    """P7: d*MSE ratios per added bit in [3, 4.2]; d*MSE*4^B <= sqrt(3)pi/2."""
    d = 128
    mses = []
    for b in (1, 2, 3, 4):
        c, _ = P.sphere_codebook_fp64(d, 1 << b)
        mses.append(d * P.codebook_mse(c, d))
    ratios = [mses[i] / mses[i + 1] for i in range(3)]
    assert all(3.0 <= r <= 4.2 for r in ratios), ratios
    for b, m in zip((1, 2, 3, 4), mses):
        assert m * 4.0 ** b <= math.sqrt(3) * math.pi / 2 + 1e-9


def test_monte_carlo_mse_matches_closed_form():
    """P7: the quantizer's empirical MSE on rotated keys equals the formula."""
    pr = P.init(64, 3, 4)
    keys = np.random.default_rng(1).standard_normal((20000, 64))
    qz = tq.quantize(pr, keys)
    emp = np.mean(qz.rnorms ** 2)          # = d * per-coordinate MSE
    c = pr.centroids
    assert abs(emp - 64 * P.codebook_mse(c, 64)) / emp < 0.015


def test_thresholds_are_midpoints_and_ties_go_up():
    pr = P.init(16, 4, 0)
    c = pr.centroids
    assert np.array_equal(pr.thresholds, (0.5 * (c[:-1] + c[1:])).astype(np.float32).astype(np.float64))
    z = pr.thresholds[None, :]
    assert np.array_equal(tq.bucketize(pr, z)[0], np.arange(1, len(c)))
    assert tq.bucketize(pr, np.array([[-0.9999]]))[0, 0] == 0
    assert tq.bucketize(pr, np.array([[0.9999]]))[0, 0] == len(c) - 1


def test_bit_split():
    """2-bit stage + 1 QJL bit = 3 bits; 3-bit stage + 1 = 4 bits."""
    assert P.init(8, 3, 0).levels == 4
    assert P.init(8, 4, 0).levels == 8
    assert P.init(8, 3, 0).code_bits == 2


# ---------------------------------------------------------------------------
# quantize / residual / signs
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d,bits", [(2, 2), (3, 3), (5, 3), (8, 2)])
def test_brute_force_nearest_codeword(d, bits):
    """P11: per-coordinate bucketize = global argmin over all (2^B)^d words."""
    pr = P.init(d, bits, 9)
    keys = np.random.default_rng(d).standard_normal((20, d))
    qz = tq.quantize(pr, keys)
    words = np.array(list(itertools.product(pr.centroids, repeat=d)))
    for i in range(len(keys)):
        dist = np.sum((words - qz.z[i][None, :]) ** 2, axis=1)
        best = words[np.argmin(dist)]
        assert np.array_equal(pr.centroids[qz.idx[i]], best)


def test_sign_convention():
    """Positive projection -> 1, negative -> 0, exactly zero -> 0."""
    pr = P.explicit(3, 2, np.eye(3), np.eye(3))
    r = np.array([[0.25, -0.25, 0.0]])
    p, beta = tq.project_signs(pr, r)
    assert beta.tolist() == [[True, False, False]]


@pytest.mark.parametrize("d,bits", [(7, 3), (128, 3), (200, 4)])
def test_isometry_identities(d, bits):
    """P8: ||u - Pi^T c[idx]|| = rho and ||k - k_hat|| = n rho."""
    pr = P.init(d, bits, 3)
    keys = np.random.default_rng(2).standard_normal((50, d)) * 3.0
    qz = tq.quantize(pr, keys)
    norms, u = tq.normalize(keys)
    recon_u = pr.centroids[qz.idx] @ pr.pi
    # Pi is float32-rounded, orthogonal to ~1e-7: the identity holds to that
    assert np.max(np.abs(np.linalg.norm(u - recon_u, axis=1) - qz.rnorms)) < 1e-6
    khat = tq.dequant_mse(pr, qz.idx, qz.norms)
    err = np.linalg.norm(keys - khat, axis=1)
    assert np.max(np.abs(err - qz.norms * qz.rnorms) / qz.norms) < 1e-6
    # with an exactly orthogonal rotation the identities are exact
    q, _ = np.linalg.qr(np.random.default_rng(4).standard_normal((d, d)))
    pe = P.Params(d, bits, 0, q, pr.g, pr.centroids, pr.thresholds)
    qe = tq.quantize(pe, keys)
    recon = pe.centroids[qe.idx] @ pe.pi
    assert np.max(np.abs(np.linalg.norm(u - recon, axis=1) - qe.rnorms)) < 1e-12


def test_zero_key_runs_literally():
    pr = P.init(16, 3, 0)
    keys = np.zeros((1, 16))
    qz = tq.quantize(pr, keys)
    assert qz.norms[0] == 0.0
    # z = 0 sits on the middle threshold: upper cell
    assert np.all(qz.idx == len(pr.centroids) // 2)
    assert np.all(tq.dequant_mse(pr, qz.idx, qz.norms) == 0.0)
    s = tq.scores(pr, np.ones((2, 16)), qz.idx, qz.beta, qz.norms, qz.rnorms)
    assert np.all(s == 0.0)


def test_scale_invariance():
    """P12: k -> 2^e k leaves codes, signs, rho identical; n scales exactly."""
    pr = P.init(64, 4, 1)
    keys = np.random.default_rng(3).standard_normal((40, 64))
    a = tq.quantize(pr, keys)
    b = tq.quantize(pr, keys * 8.0)
    assert np.array_equal(a.idx, b.idx) and np.array_equal(a.beta, b.beta)
    assert np.array_equal(a.rnorms, b.rnorms)
    assert np.array_equal(a.norms * 8.0, b.norms)


# ---------------------------------------------------------------------------
# estimator
# ---------------------------------------------------------------------------

def test_estimator_equals_dense_formula():
    """P11: s = <q, n Pi^T (c[idx] + rho sqrt(pi/2)/d G^T (2 beta - 1))>."""
    d = 6
    pr = P.init(d, 3, 5)
    rs = np.random.default_rng(6)
    keys = rs.standard_normal((9, d))
    qs = rs.standard_normal((4, d))
    qz = tq.quantize(pr, keys)
    s = tq.scores(pr, qs, qz.idx, qz.beta, qz.norms, qz.rnorms)
    for a in range(4):
        for b in range(9):
            sg = np.where(qz.beta[b], 1.0, -1.0)
            corr = qz.rnorms[b] * math.sqrt(math.pi / 2) / d * (pr.g.T @ sg)
            khat = qz.norms[b] * (pr.pi.T @ (pr.centroids[qz.idx[b]] + corr))
            assert abs(s[a, b] - qs[a] @ khat) < 1e-12 * max(1.0, abs(s[a, b]))


def test_estimator_linear_in_query():
    """P13."""
    pr = P.init(32, 3, 2)
    rs = np.random.default_rng(7)
    keys = rs.standard_normal((10, 32))
    q1, q2 = rs.standard_normal((2, 32))
    qz = tq.quantize(pr, keys)
    f = lambda q: tq.scores(pr, q[None, :], qz.idx, qz.beta, qz.norms, qz.rnorms)[0]
    assert np.allclose(f(2.5 * q1), 2.5 * f(q1), rtol=1e-12, atol=1e-12)
    assert np.allclose(f(q1 + q2), f(q1) + f(q2), rtol=1e-12, atol=1e-12)


def test_qjl_correction_unbiased_over_projections():
    """P9: averaged over Gaussian G, rho sqrt(pi/2)/d <G v, sign(G r)> -> <v, r>.

    Pi and the key are fixed; only G varies.  The spread also matches the
    closed-form variance ((pi/2) |v|^2 rho^2 - <v,r>^2) / d.
    """
    d = 48
    base = P.init(d, 3, 0)
    rs = np.random.default_rng(8)
    key = rs.standard_normal((1, d))
    q = rs.standard_normal((1, d))
    qz0 = tq.quantize(base, key)
    norms, u = tq.normalize(key)
    z = tq.rotate(base, u)
    r, rho = tq.residual(base, z, qz0.idx)
    v, _ = tq.query_transform(base, q)
    target = float(v[0] @ r[0])
    trials = 6000
    est = np.empty(trials)
    for t in range(trials):
        g = rs.standard_normal((d, d))
        pr = P.Params(d, 3, 0, base.pi, g, base.centroids, base.thresholds)
        qz = tq.quantize(pr, key)
        s = tq.scores(pr, q, qz.idx, qz.beta, qz.norms, qz.rnorms)[0, 0]
        stage1 = qz.norms[0] * float(v[0] @ pr.centroids[qz.idx[0]])
        est[t] = (s - stage1) / qz.norms[0]
    sem = est.std() / math.sqrt(trials)
    assert abs(est.mean() - target) < 4 * sem
    var_cf = (math.pi / 2 * float(v[0] @ v[0]) * rho[0] ** 2 - target ** 2) / d
    assert abs(est.var() / var_cf - 1.0) < 0.08


def test_full_estimator_unbiased_over_seeds():
    """P10: averaged over seeds of (Pi, G), the score estimates <q, k>."""
    d = 24
    rs = np.random.default_rng(9)
    key = rs.standard_normal((1, d))
    q = rs.standard_normal((1, d))
    est = np.array([tq.scores(pr, q, *(lambda z: (z.idx, z.beta, z.norms, z.rnorms))(tq.quantize(pr, key)))[0, 0]
                    for pr in (P.init(d, 2, s) for s in range(1500))])
    sem = est.std() / math.sqrt(len(est))
    assert abs(est.mean() - float(q[0] @ key[0])) < 4 * sem


# ---------------------------------------------------------------------------
# packing
# ---------------------------------------------------------------------------

def test_pack_bit_positions():
    bits = np.zeros((1, 70), dtype=bool)
    bits[0, [0, 5, 31, 32, 69]] = True
    w = tq.pack_bits(bits)
    assert w.shape == (1, 3)
    assert w[0, 0] == (1 | (1 << 5) | (1 << 31))
    assert w[0, 1] == 1
    assert w[0, 2] == (1 << 5)           # coordinate 69 = word 2, bit 5; padding 0


def test_pack_round_trip():
    rs = np.random.default_rng(1)
    idx = rs.integers(0, 8, (13, 77))
    codes = tq.pack_codes(idx, 3)
    assert codes.shape == (13, 3, 3)
    assert np.array_equal(tq.unpack_codes(codes, 77), idx)
    # plane p holds bit p of the index
    assert np.array_equal(tq.unpack_bits(codes[:, 1, :], 77), ((idx >> 1) & 1).astype(bool))
    beta = rs.random((13, 77)) > 0.5
    assert np.array_equal(tq.unpack_bits(tq.pack_bits(beta), 77), beta)


# ----------------------------------------------------------------------------
# stage 8: search (top-k per query, recall)
# ----------------------------------------------------------------------------

def test_topk_matches_brute_force_sort():
    """Against a plain sort of (-score, index) pairs, with many ties (small
    integer scores), for k below, at and above the row length."""
    rs = np.random.default_rng(5)
    for m, n, k in ((3, 1, 1), (4, 7, 3), (5, 16, 16), (2, 9, 20), (6, 33, 10)):
        s = rs.integers(-3, 4, size=(m, n)).astype(np.float64)
        idx, vals = tq.topk(s, k)
        for i in range(m):
            want = [j for _, j in sorted((-s[i, j], j) for j in range(n))][:min(k, n)]
            assert idx[i].tolist() == want
            assert vals[i].tolist() == [s[i, j] for j in want]


def test_topk_invariants():
    rs = np.random.default_rng(6)
    s = rs.standard_normal((8, 50))
    idx, vals = tq.topk(s, 10)
    assert np.array_equal(idx[:, 0], np.argmax(s, axis=1))
    assert np.all(np.diff(vals, axis=1) <= 0)
    for i in range(8):
        rest = np.setdiff1d(np.arange(50), idx[i])
        assert np.all(s[i, rest] <= vals[i, -1])
    full, _ = tq.topk(s, 50)
    assert all(sorted(r.tolist()) == list(range(50)) for r in full)


def test_recall_definitions():
    found = np.array([[0, 1, 2], [5, 6, 7]])
    exact = np.array([[2, 3, 4], [7, 6, 5]])
    assert tq.recall_at_k(found, exact) == pytest.approx((1 / 3 + 1) / 2)
    assert tq.recall_1_at_k(found, np.array([2, 9])) == 0.5
    q = np.array([[1.0, 0.0], [0.0, 1.0]])
    k = np.array([[3.0, 0.0], [0.0, 2.0], [1.0, 1.0]])
    assert np.array_equal(tq.exact_inner_products(q, k), [[3.0, 0.0, 1.0], [0.0, 2.0, 1.0]])


def test_compare_topk_flags_planted_mistakes():
    """The rule accepts the oracle's own lists and a swap at the k-th score
    within tolerance, and rejects a duplicate, a wrong order, a far miss and
    an off score (mistakes planted on the CPU)."""
    from oracle import parity
    rs = np.random.default_rng(7)
    m, n, k = 4, 40, 5
    q = rs.standard_normal((m, 8))
    norms = np.ones(n)
    s = rs.standard_normal((m, n)) * 10.0
    s[0, 7] = s[0, 3] = 50.0                         # tie at the top of row 0
    idx, vals = tq.topk(s, k)
    assert parity.compare_topk(idx, vals, s, q, norms, k).ok()
    # row 1: the (k+1)-th key within tolerance of the k-th may replace it
    order = np.argsort(-s[1], kind="stable")
    s[1, order[k]] = s[1, order[k - 1]] - 1e-4 * np.linalg.norm(q[1])
    idx, vals = tq.topk(s, k)
    near = idx.copy(); nv = vals.copy()
    near[1, -1] = order[k]; nv[1, -1] = s[1, order[k]]
    assert parity.compare_topk(near, nv, s, q, norms, k).ok()
    bad = idx.copy(); bad[2, 1] = bad[2, 0]
    assert not parity.compare_topk(bad, vals, s, q, norms, k).ok()
    swapped = idx.copy(); sv = vals.copy()
    swapped[3, [0, 1]] = swapped[3, [1, 0]]; sv[3, [0, 1]] = sv[3, [1, 0]]
    assert not parity.compare_topk(swapped, sv, s, q, norms, k).ok()
    far = idx.copy(); fv = vals.copy()
    worst = int(np.argmin(s[2])); far[2, 0] = worst; fv[2, 0] = s[2, worst]
    assert not parity.compare_topk(far, fv, s, q, norms, k).ok()
    off = vals.copy(); off[0, 2] += 1.0
    assert not parity.compare_topk(idx, off, s, q, norms, k).ok()


# ---------------------------------------------------------------------------
# reconstruction with the correction, decode attention, value blocks
# ---------------------------------------------------------------------------

def test_dequant_prod_reproduces_every_score():
    """Stage 9 is the vector whose inner product with any query is the
    (separately pinned) stage-6 estimate: linearity of the score in q."""
    pr = P.init(40, 4, 3)
    rs = np.random.default_rng(21)
    keys = rs.standard_normal((12, 40)) * 3.0
    qs = rs.standard_normal((7, 40))
    qz = tq.quantize(pr, keys)
    kt = tq.dequant_prod(pr, qz.idx, qz.beta, qz.norms, qz.rnorms)
    s = tq.scores(pr, qs, qz.idx, qz.beta, qz.norms, qz.rnorms)
    assert np.allclose(qs @ kt.T, s, rtol=1e-12, atol=1e-12)


def test_dequant_prod_unbiased_over_seeds():
    """Averaged over seeds of (Pi, G), k_tilde estimates the key itself (the
    zero-bias property, per coordinate within 4 standard errors)."""
    d = 16
    rs = np.random.default_rng(22)
    key = rs.standard_normal((1, d))
    est = []
    for seed in range(1200):
        pr = P.init(d, 2, seed)
        qz = tq.quantize(pr, key)
        est.append(tq.dequant_prod(pr, qz.idx, qz.beta, qz.norms, qz.rnorms)[0])
    est = np.array(est)
    sem = est.std(axis=0) / math.sqrt(len(est))
    assert np.all(np.abs(est.mean(axis=0) - key[0]) < 4 * sem + 1e-12)


def _attention_case(d=24, n=50, m=5, kbits=3, vbits=4, seed=23):
    prk, prv = P.init(d, kbits, seed), P.init(d, vbits, seed + 1)
    rs = np.random.default_rng(seed)
    keys = rs.standard_normal((n, d)) * np.exp(0.5 * rs.standard_normal((n, 1)))
    vals = rs.standard_normal((n, d))
    qs = rs.standard_normal((m, d))
    kz, vz = tq.quantize(prk, keys), tq.quantize(prv, vals)
    return prk, prv, qs, kz, vz


def test_attention_equals_library_sdpa():
    """Stage 10 against torch's scaled_dot_product_attention (float64, CPU)
    over the explicit reconstructions: keys k_tilde (stage 9), values v_hat
    (stage 7); lse against scipy's logsumexp."""
    import torch
    from scipy.special import logsumexp
    prk, prv, qs, kz, vz = _attention_case()
    scale = 0.37
    o, lse = tq.attention(prk, prv, qs, kz.idx, kz.beta, kz.norms, kz.rnorms, vz.idx, vz.norms, scale)
    kt = tq.dequant_prod(prk, kz.idx, kz.beta, kz.norms, kz.rnorms)
    vh = tq.dequant_mse(prv, vz.idx, vz.norms)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qs)[None], torch.from_numpy(kt)[None], torch.from_numpy(vh)[None], scale=scale)[0].numpy()
    assert np.allclose(o, ref, rtol=1e-10, atol=1e-12)
    assert np.allclose(lse, logsumexp(scale * (qs @ kt.T), axis=1), rtol=1e-12, atol=1e-12)


def test_attention_special_cases():
    """Closed forms: a zero query weighs every token alike (o = mean of the
    reconstructed values, lse = log n); one token gives its value; a large
    scale picks the best-scoring token; no tokens give o = 0, lse = -inf;
    the order of the tokens does not matter."""
    prk, prv, qs, kz, vz = _attention_case()
    args = lambda sl: (kz.idx[sl], kz.beta[sl], kz.norms[sl], kz.rnorms[sl], vz.idx[sl], vz.norms[sl])
    every = slice(None)
    vh = tq.dequant_mse(prv, vz.idx, vz.norms)
    o, lse = tq.attention(prk, prv, np.zeros((1, prk.d)), *args(every), 0.5)
    assert np.allclose(o[0], vh.mean(axis=0), rtol=1e-12, atol=1e-12)
    assert abs(lse[0] - math.log(len(vh))) < 1e-12
    o, lse = tq.attention(prk, prv, qs, *args(slice(3, 4)), 0.5)
    assert np.allclose(o, vh[3][None, :].repeat(len(qs), 0), rtol=1e-12, atol=1e-12)
    s = tq.scores(prk, qs, kz.idx, kz.beta, kz.norms, kz.rnorms)
    o, _ = tq.attention(prk, prv, qs, *args(every), 1e4)
    assert np.allclose(o, vh[np.argmax(s, axis=1)], rtol=1e-9, atol=1e-9)
    o, lse = tq.attention(prk, prv, qs, *args(slice(0, 0)), 0.5)
    assert np.all(o == 0.0) and np.all(np.isneginf(lse))
    perm = np.random.default_rng(5).permutation(len(vh))
    o1, l1 = tq.attention(prk, prv, qs, *args(every), 0.5)
    o2, l2 = tq.attention(prk, prv, qs, *args(perm), 0.5)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-12) and np.allclose(l1, l2, rtol=1e-12, atol=1e-12)


def test_pack_values_bit_positions():
    """Token-blocked value layout, worked by hand.  d = 50: W = 2 words, one
    group of G = 2.  B = 2 (E = 4): token 33 (block 1, octet 0, t = 1) with
    index 0b10 at coordinate 37 (r = 37) sets plane-1 bit (1 div 4) * 8 +
    1 * 4 + 1 = 5 of X at byte ((37 mod 16) + 0) * 8 + (37 div 16) * 2 = 44
    of block 1: byte 44 = 0x20, nothing else.  Token 14 (block 0, octet 1,
    t = 6) with index 0b01 at coordinate 3: plane-0 bit (6 div 4) * 8 + 0 +
    2 = 10 of X at byte (3 + 16) * 8 + 0 = 152: byte 153 = 0x04."""
    idx = np.zeros((40, 50), dtype=np.int64)
    idx[33, 37] = 2
    raw = tq.pack_values(idx, 2).view(np.uint8).reshape(2, 512)
    assert raw[1, 44] == 0x20 and np.count_nonzero(raw) == 1
    idx = np.zeros((40, 50), dtype=np.int64)
    idx[14, 3] = 1
    raw = tq.pack_values(idx, 2).view(np.uint8).reshape(2, 512)
    assert raw[0, 153] == 0x04 and np.count_nonzero(raw) == 1
    # B = 3 (E = 2), d = 200: W = 7, a full group then G = 3 from byte
    # 512 * 3 = 1536; coordinate 130 is r = 2 of group 1, octet 2: X at
    # 1536 + (2 + 32) * 18 + 0 = 2148; token 8*2 + 5 (t = 5) plane 2 ->
    # bit 2 * 6 + 2 * 2 + 1 = 17 -> byte 2150 bit 1
    slot = tq.value_slot(200, 3)
    assert slot[130, 2] == 2148
    idx = np.zeros((32, 200), dtype=np.int64)
    idx[21, 130] = 4
    raw = tq.pack_values(idx, 3).view(np.uint8).reshape(-1)
    assert raw[2150] == 0x02 and np.count_nonzero(raw) == 1
    # slots tile the block without overlap, B bytes each
    for d, b in ((200, 3), (50, 2), (128, 4), (33, 1)):
        s = tq.value_slot(d, b)
        cover = sorted((s[:, :, None] + np.arange(b)[None, None, :]).ravel().tolist())
        assert cover == list(range(4 * b * 32 * tq.words_per_plane(d)))
    rs = np.random.default_rng(3)
    for n, d, b in ((77, 45, 3), (40, 200, 2), (33, 128, 4), (70, 64, 1), (65, 33, 2)):
        idx = rs.integers(0, 1 << b, (n, d))
        assert np.array_equal(tq.unpack_values(tq.pack_values(idx, b), n, d), idx)


# ---------------------------------------------------------------------------
# randomized Hadamard rotation
# ---------------------------------------------------------------------------

def test_hadamard_rotation_definition_and_pages_example():
    """The randomized Hadamard rotation: scipy's Sylvester matrix against the
    definition (-1)^popcount(i & j); orthogonal to float32 rounding; at d = 4
    the unsigned matrix is the pages' 4-D example (H_4 / 2, the golden
    fixture), so 10 e_1 rotates to +-5 in every coordinate; any one-axis
    vector spreads evenly (every |entry| = 1/sqrt(d))."""
    for d in (2, 4, 16, 128):
        pi = P.hadamard_rotation(d, 11)
        sigma = np.sign(pi[0])                    # row 0 of H is all ones
        h = np.sqrt(d) * pi * sigma[None, :]
        ref = np.array([[(-1.0) ** bin(i & j).count("1") for j in range(d)] for i in range(d)])
        assert np.allclose(h, ref, rtol=1e-6, atol=0)
        assert np.max(np.abs(pi @ pi.T - np.eye(d))) < 4 * d * 2.0 ** -24
        assert np.allclose(np.abs(pi), 1.0 / np.sqrt(d), rtol=1e-7)
    g = _golden("polarquant_4d_example.json")
    pi = P.hadamard_rotation(4, 11)
    unsigned = pi * np.sign(pi[0])[None, :]
    assert np.array_equal(unsigned, np.array(g["rotation"]))
    z = unsigned @ np.array(g["input"])
    assert np.array_equal(z, np.array(g["expected"]))


def test_projection_matrix_is_the_nearest_float16_of_each_draw():
    """G keeps the projection stream's N(0, 1) draws to float16 precision:
    every entry is a float16 value and no float16 value lies closer to the
    draw (ties at exactly half a spacing allowed); the rounding leaves the
    law standard normal (KS), and in the float16 normal range keeps every
    draw's sign and moves it by at most 2^-11 of itself."""
    for d, seed in ((64, 3), (200, 0)):
        raw = P.gaussian_projection(d, seed)
        g = P.projection_matrix(d, seed)
        h = g.astype(np.float16)
        assert np.array_equal(h.astype(np.float64), g)
        up = np.nextafter(h, np.float16(np.inf)).astype(np.float64)
        dn = np.nextafter(h, np.float16(-np.inf)).astype(np.float64)
        err = np.abs(g - raw)
        assert np.all(err <= np.abs(up - raw)) and np.all(err <= np.abs(dn - raw))
        normal = np.abs(raw) >= 2.0 ** -14  # float16 normal range
        assert np.all(np.sign(g[normal]) == np.sign(raw[normal]))
        assert np.max(err[normal] / np.abs(raw[normal])) <= 2.0 ** -11
        assert stats.kstest(g.ravel(), "norm").pvalue > 1e-3


def test_hadamard_signs_balanced_and_seeded():
    """Stream-2 signs: +-1 with mean within 4 standard errors of 0; distinct
    seeds give distinct sign vectors, the same seed the same one."""
    s = rng.signs(3, 2, 20000)
    assert set(np.unique(s)) == {-1.0, 1.0}
    assert abs(s.mean()) < 4 / np.sqrt(len(s))
    assert np.array_equal(P.hadamard_rotation(64, 5), P.hadamard_rotation(64, 5))
    assert not np.array_equal(P.hadamard_rotation(64, 5), P.hadamard_rotation(64, 6))


def test_hadamard_quantizer_mse_close_to_haar():
    """With the randomized Hadamard rotation the stage-1 distortion of random
    unit vectors stays near the Haar rotation's closed form (d MSE at
    d = 128, 3 bits: 0.0340 for the coordinate law the codebook is built
    for); the rotation only approximates that law, so a 10 % band."""
    d = 128
    pr = P.init_hadamard(d, 4, 2)
    rs = np.random.default_rng(4)
    x = rs.standard_normal((4000, d))
    qz = tq.quantize(pr, x)
    mse = float(np.mean(qz.rnorms ** 2))
    assert abs(mse / 0.0340 - 1.0) < 0.1, mse


# ---------------------------------------------------------------------------
# fractional widths (stage 11)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d,bits,hi", [(40, 2, 16), (128, 3, 64), (33, 2, 33), (50, 4, 7)])
def test_split_indices_are_the_two_plain_quantizers(d, bits, hi):
    """Stage 11 against two independently pinned quantizers of the same
    seed: coordinates below hi carry the (bits + 1)-bit handle's index, the
    rest the bits-bit handle's, and the residual / scores / reconstructions
    use the matching levels (the finer set's levels are the bits + 1
    handle's, the coarse set's the bits handle's)."""
    seed = 5
    pr = P.init_split(d, bits, hi, seed)
    fine, base = P.init(d, bits + 1, seed), P.init(d, bits, seed)
    assert np.array_equal(pr.centroids_hi, fine.centroids) and np.array_equal(pr.centroids, base.centroids)
    rs = np.random.default_rng(d + hi)
    keys = rs.standard_normal((60, d)) * 2.0
    qz = tq.quantize(pr, keys)
    qf, qb = tq.quantize(fine, keys), tq.quantize(base, keys)
    assert np.array_equal(qz.idx[:, :hi], qf.idx[:, :hi])
    assert np.array_equal(qz.idx[:, hi:], qb.idx[:, hi:])
    # the residual takes each coordinate's own level
    r = np.concatenate([qf.z[:, :hi] - fine.centroids[qf.idx[:, :hi]],
                        qb.z[:, hi:] - base.centroids[qb.idx[:, hi:]]], axis=1)
    assert np.allclose(qz.rnorms, np.sqrt((r * r).sum(axis=1)), rtol=1e-13)
    # stage-1 reconstruction: Pi^T of the same level vector
    khat = tq.dequant_mse(pr, qz.idx, qz.norms)
    want = qz.norms[:, None] * (np.concatenate([fine.centroids[qz.idx[:, :hi]], base.centroids[qz.idx[:, hi:]]],
                                               axis=1) @ pr.pi)
    assert np.allclose(khat, want, rtol=1e-12, atol=1e-12)
    # the corrected reconstruction reproduces every score (linearity in q)
    qs = rs.standard_normal((4, d))
    kt = tq.dequant_prod(pr, qz.idx, qz.beta, qz.norms, qz.rnorms)
    s = tq.scores(pr, qs, qz.idx, qz.beta, qz.norms, qz.rnorms)
    assert np.allclose(qs @ kt.T, s, rtol=1e-11, atol=1e-11)


def test_split_mse_interpolates_the_closed_forms():
    """Empirical ||z - c[idx]||^2 over many rotated keys equals
    hi * m(2L) + (d - hi) * m(L), m the per-coordinate closed form of each
    level set: 2.5 bits lands between the 2- and 3-bit errors."""
    d, bits, hi = 64, 2, 32
    pr = P.init_split(d, bits, hi, 4)
    keys = np.random.default_rng(2).standard_normal((20000, d))
    qz = tq.quantize(pr, keys)
    emp = np.mean(qz.rnorms ** 2)
    m_fine, m_base = P.codebook_mse(pr.centroids_hi, d), P.codebook_mse(pr.centroids, d)
    want = hi * m_fine + (d - hi) * m_base
    assert abs(emp - want) / want < 0.015
    assert d * m_fine < emp < d * m_base


def test_split_estimator_unbiased_over_seeds():
    """The score with fractional widths still estimates <q, k> without bias
    (averaged over seeds of (Pi, G))."""
    d = 24
    rs = np.random.default_rng(19)
    key = rs.standard_normal((1, d))
    q = rs.standard_normal((1, d))
    est = []
    for seed in range(1500):
        pr = P.init_split(d, 2, 12, seed)
        z = tq.quantize(pr, key)
        est.append(tq.scores(pr, q, z.idx, z.beta, z.norms, z.rnorms)[0, 0])
    est = np.array(est)
    sem = est.std() / math.sqrt(len(est))
    assert abs(est.mean() - float(q[0] @ key[0])) < 4 * sem


def test_split_pack_bit_positions():
    """Hand-worked packing: d = 40 (W = 2), B = 1, hi = 8: plane 0 over all
    40 coordinates in words 0-1, then plane 1 over coordinates 0-7 in word
    2; the storage is B d + hi index bits per key."""
    idx = np.zeros((1, 40), dtype=np.int64)
    idx[0, 0] = 3      # plane 0 word 0 bit 0, plane 1 bit 0
    idx[0, 7] = 2      # plane 1 bit 7 only
    idx[0, 33] = 1     # plane 0 word 1 bit 1
    codes = tq.pack_codes_split(idx, 1, 8)
    assert codes.shape == (1, 3)
    assert codes[0].tolist() == [1, 1 << 1, 1 | (1 << 7)]
    assert np.array_equal(tq.unpack_codes_split(codes, 40, 1, 8), idx)
    rs = np.random.default_rng(3)
    big = rs.integers(0, 4, (9, 77))
    big[:, 45:] &= 1
    c = tq.pack_codes_split(big, 1, 45)
    assert c.shape == (9, 3 + 2)
    assert np.array_equal(tq.unpack_codes_split(c, 77, 1, 45), big)
    # hi = 0 is the plain layout, flattened
    plain = rs.integers(0, 8, (4, 70))
    assert np.array_equal(tq.pack_codes_split(plain, 3, 0), tq.pack_codes(plain, 3).reshape(4, -1))


# ---------------------------------------------------------------------------
# the parity rules themselves (oracle.parity), with mistakes planted on the CPU
# ---------------------------------------------------------------------------

def _bisect(f, lo, hi, iters=200):
    """Root of a monotone scalar function between lo and hi (float64)."""
    flo = f(lo)
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        fm = f(mid)
        if (fm > 0) == (flo > 0):
            lo, flo = mid, fm
        else:
            hi = mid
    return 0.5 * (lo + hi)


def _plant_z(pr, key, j, target):
    """key + a Pi_j so that the oracle's z_j equals target (found by
    bisection through the oracle's own normalize + rotate)."""
    row = pr.pi[j]
    zj = lambda a: tq.rotate(pr, tq.normalize((key + a * row)[None, :])[1])[0, j] - target
    a = _bisect(zj, -0.3 * np.linalg.norm(key), 0.3 * np.linalg.norm(key))
    return key + a * row


def _plant_p(pr, key, target):
    """key moved along Pi^T G_j, for the j of its smallest |p_j|, so that the
    oracle's p_j equals target; None when a code changes on the way."""
    base = tq.quantize(pr, key[None, :])
    j = int(np.argmin(np.abs(base.p[0])))
    direction = pr.pi.T @ pr.g[j]
    direction /= np.linalg.norm(direction)
    pj = lambda a: tq.quantize(pr, (key + a * direction)[None, :]).p[0, j] - target
    span = 0.05 * np.linalg.norm(key)
    if (pj(-span) > 0) == (pj(span) > 0):
        return None, j
    moved = key + _bisect(pj, -span, span) * direction
    if not np.array_equal(tq.quantize(pr, moved[None, :]).idx, base.idx):
        return None, j
    return moved, j


def _packed(pr, qz):
    codes, signs, norms, rnorms = tq.pack(pr, qz)
    return codes.copy(), signs.copy(), norms.astype(np.float32), rnorms.astype(np.float32)


def _planted_case():
    """2000 keys at d = 32, 3 bits (128 000 decisions, so one mismatch is a
    rate of 7.8e-6): key 0 has z_3 3e-7 above threshold 1; key a has one
    p_j = 3e-6 (outside |p| < 1e-6, inside |p| / sqrt(d) < 1e-6) and key b
    one p_j = 4e-7 (inside both windows).  Returns the keys' positions."""
    pr = P.init(32, 3, 5)
    rs = np.random.default_rng(55)
    keys = rs.standard_normal((2000, 32))
    t = pr.thresholds[1]
    keys[0] = _plant_z(pr, keys[0], 3, t + 3e-7)
    planted = []
    for target in (3e-6, 4e-7):
        for i in range(1 + len(planted) * 100, 2000):
            moved, j = _plant_p(pr, keys[i], target)
            if moved is not None:
                keys[i] = moved
                planted.append((i, j))
                break
    qz = tq.quantize(pr, keys)
    assert 0 < qz.z[0, 3] - t < 1e-6
    (a, ja), (b, jb) = planted
    assert abs(qz.p[a, ja] - 3e-6) < 1e-10 and abs(qz.p[b, jb] - 4e-7) < 1e-10
    return pr, keys, qz, planted


def test_compare_quantize_accepts_the_oracle_and_in_window_flips():
    """The oracle's own packed output passes with no mismatch.  A code
    flipped inside the window passes when the key's signs and rho are the
    oracle's for the flipped code (the cascade), and is counted; a sign
    flipped inside |p| < 1e-6 passes and is counted."""
    from oracle import parity
    pr, keys, qz, ((a, ja), (b, jb)) = _planted_case()
    rep = parity.compare_quantize(pr, qz, *_packed(pr, qz))
    assert rep.ok() and rep.code_mismatch == rep.sign_mismatch == rep.cascade_keys == 0
    assert rep.elements == 2 * 2000 * 32

    idx = qz.idx.copy()
    idx[0, 3] -= 1                                 # the lower cell, 3e-7 away
    ref = parity.reference_for_codes(pr, qz, idx)
    assert not np.array_equal(ref.beta[0], qz.beta[0]) and ref.rnorms[0] != qz.rnorms[0]
    assert np.array_equal(ref.beta[1:], qz.beta[1:])
    rep = parity.compare_quantize(pr, qz, *_packed(pr, ref))
    assert rep.ok(), rep
    assert rep.code_mismatch == 1 and rep.code_bad == 0 and rep.cascade_keys == 1 and rep.sign_mismatch == 0

    beta = qz.beta.copy()
    beta[b, jb] = ~beta[b, jb]
    rep = parity.compare_quantize(pr, qz, *_packed(pr, tq.Quantized(qz.idx, beta, qz.norms, qz.rnorms, qz.z, qz.p)))
    assert rep.ok() and rep.sign_mismatch == 1 and rep.sign_bad == 0 and rep.decision_keys == 1
    # that one in-window sign moves the key's scores by more than the score
    # bound for some queries; the end-to-end reference is the estimator on
    # the library's decisions, which the scores computed from them meet
    q = np.random.default_rng(9).standard_normal((64, 32))
    lib = tq.scores(pr, q, qz.idx[b:b + 1], beta[b:b + 1], qz.norms[b:b + 1], qz.rnorms[b:b + 1])
    own = tq.scores(pr, q, qz.idx[b:b + 1], qz.beta[b:b + 1], qz.norms[b:b + 1], qz.rnorms[b:b + 1])
    assert parity.score_violations(lib, own, q, qz.norms[b:b + 1])[0] > 0
    ref = parity.e2e_scores(pr, rep, q, qz.norms[b:b + 1], slice(b, b + 1))
    assert parity.score_violations(lib, ref, q, qz.norms[b:b + 1]) == (0, 0.0)


def test_compare_quantize_rejects_planted_mistakes():
    """Each of these makes the comparison fail: a flipped code whose key
    keeps the unflipped code's signs (the cascade not followed), a code
    flipped outside the window, a sign flipped outside |p| < 1e-6 (also when
    it is inside the wider |p| / sqrt(d) window, which is only reported), a
    NaN / infinite / off norm or rho, a set padding bit, and in-window
    mismatches above 1e-5 of the decisions."""
    from oracle import parity
    pr, keys, qz, ((a, ja), (b, jb)) = _planted_case()

    def run(codes=None, signs=None, norms=None, rnorms=None, params=pr, q=qz):
        c, s, n, r = _packed(params, q)
        return parity.compare_quantize(params, q, *(x if x is not None else y
                                                   for x, y in zip((codes, signs, norms, rnorms), (c, s, n, r))))

    idx = qz.idx.copy()
    idx[0, 3] -= 1
    stale = tq.pack(pr, tq.Quantized(idx, qz.beta, qz.norms, qz.rnorms, qz.z, qz.p))
    rep = run(codes=stale[0])
    assert not rep.ok() and rep.sign_bad > 0 and rep.cascade_keys == 1

    far = int(np.argmax(np.min(np.abs(qz.z[5, :, None] - pr.thresholds[None, :]), axis=1)))
    idx = qz.idx.copy()
    idx[5, far] = (idx[5, far] + 1) % 4
    ref = parity.reference_for_codes(pr, qz, idx)
    rep = run(codes=_packed(pr, ref)[0], signs=_packed(pr, ref)[1], rnorms=_packed(pr, ref)[3])
    assert not rep.ok() and rep.code_bad == 1 and "code" in rep.worst

    beta = qz.beta.copy()
    beta[a, ja] = ~beta[a, ja]                     # |p| = 3e-6: outside 1e-6, inside 1e-6 sqrt(32)
    rep = run(signs=tq.pack_bits(beta))
    assert not rep.ok() and rep.sign_bad == 1 and rep.sign_bad_normalized == 0
    beta = qz.beta.copy()
    far = int(np.argmax(np.abs(qz.p[9])))
    beta[9, far] = ~beta[9, far]
    rep = run(signs=tq.pack_bits(beta))
    assert not rep.ok() and rep.sign_bad == 1 and rep.sign_bad_normalized == 1

    for bad in (np.nan, np.inf):
        n = qz.norms.astype(np.float32)
        n[11] = bad
        rep = run(norms=n)
        assert not rep.ok() and rep.norm_bad == 1 and rep.nonfinite == 1
        r = qz.rnorms.astype(np.float32)
        r[12] = bad
        rep = run(rnorms=r)
        assert not rep.ok() and rep.rnorm_bad == 1
    n = qz.norms.astype(np.float32)
    n[13] = qz.norms[13] * (1 + 2 * 32 * 2.0 ** -24)
    assert run(norms=n).norm_bad == 1
    r = qz.rnorms.astype(np.float32)
    r[14] = qz.rnorms[14] + 3 * (np.sqrt(32) * 1e-6 + 32 * 2.0 ** -24 * qz.rnorms[14])
    assert run(rnorms=r).rnorm_bad == 1
    # all-NaN outputs, as from a kernel that never wrote them
    rep = run(norms=np.full(2000, np.nan, np.float32), rnorms=np.full(2000, np.nan, np.float32))
    assert not rep.ok() and rep.norm_bad == 2000 and rep.rnorm_bad == 2000

    # a padding bit past d (d = 30: the top two bits of the last word)
    pr30 = P.init(30, 3, 5)
    q30 = tq.quantize(pr30, keys[:, :30])
    c, s, n, r = _packed(pr30, q30)
    s[4, 0] |= np.uint32(1 << 31)
    assert parity.compare_quantize(pr30, q30, c, s, n, r).padding_bad == 1
    c[6, 1, 0] |= np.uint32(1 << 30)
    assert not parity.compare_quantize(pr30, q30, c, *_packed(pr30, q30)[1:]).ok()

    # the rate: the in-window flip of key 0 is 1 of 2 * 10 * 32 decisions
    sub = tq.quantize(pr, keys[:10])
    idx = sub.idx.copy()
    idx[0, 3] -= 1
    ref = parity.reference_for_codes(pr, sub, idx)
    rep = parity.compare_quantize(pr, sub, *_packed(pr, ref))
    assert rep.code_bad == 0 and rep.sign_bad == 0 and rep.mismatch_rate > 1e-5 and not rep.ok()


def test_score_and_reconstruction_rules_reject_planted_mistakes():
    """score_violations and dequant_violations count an error of twice the
    tolerance, a NaN and an infinity as violations (worst ratio inf for the
    non-finite ones), and pass the oracle's own values and an error of half
    the tolerance."""
    from oracle import parity
    pr = P.init(24, 3, 2)
    rs = np.random.default_rng(8)
    keys = rs.standard_normal((40, 24)) * 2.0
    q = rs.standard_normal((3, 24))
    qz = tq.quantize(pr, keys)
    s = tq.scores(pr, q, qz.idx, qz.beta, qz.norms, qz.rnorms)
    tol = 1e-3 * np.linalg.norm(q, axis=1)[:, None] * qz.norms[None, :]
    assert parity.score_violations(s, s, q, qz.norms) == (0, 0.0)
    half = s + 0.5 * tol
    bad, worst = parity.score_violations(half, s, q, qz.norms)
    assert bad == 0 and worst == pytest.approx(0.5)
    for planted, ratio in ((s[1, 7] + 2 * tol[1, 7], 2.0), (np.nan, np.inf), (np.inf, np.inf), (-np.inf, np.inf)):
        x = s.copy()
        x[1, 7] = planted
        bad, worst = parity.score_violations(x, s, q, qz.norms)
        assert bad == 1 and worst == pytest.approx(ratio)
        keep = np.ones(40, dtype=bool)
        keep[7] = False
        assert parity.score_violations(x, s, q, qz.norms, keep=keep)[0] == 0
    assert parity.score_violations(np.full_like(s, np.nan), s, q, qz.norms)[0] == s.size

    kh = tq.dequant_mse(pr, qz.idx, qz.norms)
    assert parity.dequant_violations(kh, kh) == (0, 0.0)
    e = np.zeros(24)
    e[0] = 1.0
    x = kh.copy()
    x[3] += 2e-5 * np.linalg.norm(kh[3]) * e
    bad, worst = parity.dequant_violations(x, kh)
    assert bad == 1 and worst == pytest.approx(2.0)
    x = kh.copy()
    x[4] += 0.5e-5 * np.linalg.norm(kh[4]) * e
    assert parity.dequant_violations(x, kh)[0] == 0
    for planted in (np.nan, np.inf):
        x = kh.copy()
        x[5, 2] = planted
        bad, worst = parity.dequant_violations(x, kh)
        assert bad == 1 and worst == np.inf
    assert parity.dequant_violations(np.full_like(kh, np.nan), kh)[0] == 40


# ---------------------------------------------------------------------------
# the recursive polar-angle variant of stage 1 (oracle.polar)
# ---------------------------------------------------------------------------

def test_polar_decompose_hand_examples_and_round_trip():
    """Hand-worked decompositions (level-1 angle of the pair (0, 1) is pi/2,
    of (1, 0) is 0, of (0, -1) is 3 pi/2; the top angle compares the two
    halves' lengths), d - 1 angles, top radius = ||z||, and compose inverts
    decompose."""
    from oracle import polar as PL
    z = np.array([[1.0, 0.0, 0.0, 0.0], [0.0, 0.0, 0.0, 1.0], [0.0, -1.0, 0.0, 0.0], [0.6, 0.0, 0.0, 0.8]])
    ang, r = PL.decompose(z)
    assert [a.shape[1] for a in ang] == [2, 1]
    assert np.allclose(ang[0], [[0.0, 0.0], [0.0, np.pi / 2], [3 * np.pi / 2, 0.0], [0.0, np.pi / 2]])
    assert np.allclose(ang[1][:, 0], [0.0, np.pi / 2, 0.0, np.arctan2(0.8, 0.6)])
    assert np.allclose(r, 1.0)
    rs = np.random.default_rng(31)
    for d in (2, 8, 64, 256):
        x = rs.standard_normal((20, d)) * 3.0
        ang, r = PL.decompose(x)
        assert sum(a.shape[1] for a in ang) == d - 1
        assert np.allclose(r, np.linalg.norm(x, axis=1), rtol=1e-14)
        assert np.allclose(PL.compose(ang, r), x, atol=1e-12)
        assert np.all((ang[0] >= 0) & (ang[0] < 2 * np.pi))
        assert all(np.all((a >= 0) & (a <= np.pi / 2)) for a in ang[1:])


def test_polar_angle_laws():
    """For uniformly random unit vectors (d = 64), level-1 angles are uniform
    on [0, 2 pi) and a level-l angle has the law sin^2 psi ~ Beta(m/2, m/2),
    m = 2^(l-1) (Kolmogorov-Smirnov; the CDF is checked against direct
    quadrature of the density)."""
    from oracle import polar as PL
    rs = np.random.default_rng(32)
    x = rs.standard_normal((4000, 64))
    ang, _ = PL.decompose(x / np.linalg.norm(x, axis=1, keepdims=True))
    assert stats.kstest(ang[0].ravel(), stats.uniform(0, 2 * np.pi).cdf).pvalue > 1e-3
    for lvl in range(2, 7):
        m = 1 << (lvl - 1)
        assert stats.kstest(ang[lvl - 1].ravel(), lambda p: PL.angle_cdf(p, m)).pvalue > 1e-3
        for p in (0.3, np.pi / 4, 1.2):
            assert PL.angle_cdf(p, m) == pytest.approx(integrate.quad(lambda s: PL.angle_pdf(s, m), 0, p)[0],
                                                       rel=1e-9, abs=1e-12)


def test_polar_codebooks_closed_forms_and_fixed_point():
    """m = 2 (density sin 2 psi on [0, pi/2]) with 2 levels: the threshold
    is pi/4 and the levels are 1/2 and pi/2 - 1/2 (closed form of the
    conditional means).  Other laws: every level is the conditional mean of
    its cell, with the mass from the Beta CDF of sin^2 psi (a second route to
    the mass) and the moment by quadrature; levels are symmetric about pi/4.
    Level 1 of a handle is the uniform quantizer of the circle."""
    from oracle import polar as PL
    c = PL.level_codebook_fp64(2, 2)
    assert c == pytest.approx([0.5, np.pi / 2 - 0.5], abs=1e-12)
    for m, levels in ((2, 4), (8, 4), (64, 8), (512, 2)):
        c = PL.level_codebook_fp64(m, levels)
        assert np.allclose(c + c[::-1], np.pi / 2, atol=1e-13)
        t = np.concatenate(([0.0], 0.5 * (c[:-1] + c[1:]), [np.pi / 2]))
        for i in range(levels):
            mass = PL.angle_cdf(t[i + 1], m) - PL.angle_cdf(t[i], m)
            mom = integrate.quad(lambda s: s * PL.angle_pdf(s, m), t[i], t[i + 1], epsrel=1e-13, limit=200)[0]
            assert mom / mass == pytest.approx(c[i], rel=1e-9)
    pp = PL.init_polar(16, 3, 0)
    assert np.allclose(pp.centroids[0], (np.arange(4) + 0.5) * np.pi / 2, rtol=1e-7)
    assert np.allclose(pp.thresholds[0], np.arange(1, 4) * np.pi / 2, rtol=1e-7)
    assert len(pp.centroids) == 4 and all(len(x) == 4 for x in pp.centroids)


def test_polar_d2_mse_closed_form():
    """d = 2: one uniform angle, L levels on the circle; the squared error of
    the unit vector is 2 - 2 cos(e) with e uniform on [-pi/L, pi/L], so its
    mean is 2 - 2 sin(pi/L) / (pi/L)."""
    from oracle import polar as PL
    for bits in (2, 3, 4):
        pp = PL.init_polar(2, bits, 1)
        L = 1 << (bits - 1)
        th = (np.arange(400000) + 0.5) * (2 * np.pi / 400000)   # midpoint rule over the circle
        z = np.stack([np.cos(th), np.sin(th)], axis=1)
        ang, _ = PL.decompose(z)
        zh = PL.reconstruct(pp, PL.quantize_angles(pp, ang))
        mse = np.mean(np.sum((z - zh) ** 2, axis=1))
        h = np.pi / L
        assert mse == pytest.approx(2 - 2 * np.sin(h) / h, rel=1e-6)


def test_polar_scores_equal_dense_formula_and_qjl_unbiased():
    """The polar score equals <q, n Pi^T (z_hat + rho sqrt(pi/2)/d G^T s)>
    with explicit matrices (catches a transposed operand), the slot packing
    round-trips, and the QJL term averaged over 6000 Gaussian G estimates
    <q, Pi^T r> (zero bias) within 4 standard errors."""
    from oracle import polar as PL
    pp = PL.init_polar(16, 3, 4)
    rs = np.random.default_rng(34)
    keys = rs.standard_normal((9, 16)) * 2.0
    q = rs.standard_normal((5, 16))
    pq = PL.quantize(pp, keys)
    s = PL.scores(pp, q, pq.codes, pq.beta, pq.norms, pq.rnorms)
    sg = np.where(pq.beta, 1.0, -1.0)
    kt = pq.norms[:, None] * ((pq.zhat + (pq.rnorms * tq.QJL_CONST / 16)[:, None] * (sg @ pp.g)) @ pp.pi)
    assert np.allclose(s, q @ kt.T, rtol=1e-12, atol=1e-12)
    sl = PL.slots(pq.codes)
    assert sl.shape == (9, 16) and np.all(sl[:, 15] == 0)
    assert all(np.array_equal(a, b) for a, b in zip(PL.unslot(sl, 16), pq.codes))
    # zero bias of the QJL term over projections
    u = keys[0] / np.linalg.norm(keys[0])
    z = pp.pi @ u
    ang, _ = PL.decompose(z[None, :])
    r = z - PL.reconstruct(pp, PL.quantize_angles(pp, ang))[0]
    v = pp.pi @ q[0]
    est = []
    for _ in range(6000):
        g = rs.standard_normal((16, 16))
        est.append(np.linalg.norm(r) * tq.QJL_CONST / 16 * (g @ v) @ np.where(g @ r > 0, 1.0, -1.0))
    est = np.array(est)
    assert abs(est.mean() - v @ r) < 4 * est.std() / np.sqrt(len(est))


def test_compare_quantize_polar_rules():
    """The polar rule passes the oracle's own packed output and rejects a
    code changed far from its boundary, a flipped sign far from 0, a NaN
    norm and a set unused slot; a code changed at an angle within 1e-6 of a
    boundary passes when the key's signs and rho follow the changed code."""
    from oracle import parity
    from oracle import polar as PL
    pp = PL.init_polar(32, 3, 6)
    rs = np.random.default_rng(35)
    keys = rs.standard_normal((3000, 32))
    pq = PL.quantize(pp, keys)
    codes = tq.pack_codes(PL.slots(pq.codes), 2)
    signs = tq.pack_bits(pq.beta)
    n32, r32 = pq.norms.astype(np.float32), pq.rnorms.astype(np.float32)
    rep = parity.compare_quantize_polar(pp, pq, codes, signs, n32, r32)
    assert rep.ok() and rep.code_mismatch == rep.sign_mismatch == 0, rep
    dist = parity.polar_angle_distance(pp, pq.angles)
    k, j = np.unravel_index(np.argmax(np.where(np.isfinite(dist), dist, -1)), dist.shape)
    sl = PL.slots(pq.codes)
    sl[k, j] = (sl[k, j] + 1) % 4
    assert parity.compare_quantize_polar(pp, pq, tq.pack_codes(sl, 2), signs, n32, r32).code_bad == 1
    beta = pq.beta.copy()
    far = int(np.argmax(np.abs(pq.p[7])))
    beta[7, far] = ~beta[7, far]
    assert parity.compare_quantize_polar(pp, pq, codes, tq.pack_bits(beta), n32, r32).sign_bad == 1
    bad = n32.copy()
    bad[3] = np.nan
    assert not parity.compare_quantize_polar(pp, pq, codes, signs, bad, r32).ok()
    sl = PL.slots(pq.codes)
    sl[5, 31] = 1
    assert parity.compare_quantize_polar(pp, pq, tq.pack_codes(sl, 2), signs, n32, r32).padding_bad == 1
    # an in-window change: plant an angle 3e-7 above a level-2 threshold
    # through the inverse transform, flip its code to the lower cell and give
    # the key the signs and rho of the changed code
    z = pq.z[0].copy()
    ang, r = PL.decompose(z[None, :])
    t = pp.thresholds[1][1]
    ang[1][0, 3] = t + 3e-7
    key = PL.compose(ang, r)[0] @ pp.pi   # Pi^T z (Pi is orthogonal to 1e-7)
    pq1 = PL.quantize(pp, key[None, :])
    d1 = parity.polar_angle_distance(pp, pq1.angles)[0, 16 + 3]
    assert d1 < 1e-6, d1
    sl = PL.slots(pq1.codes)
    sl[0, 16 + 3] -= 1
    changed = PL.unslot(sl, 32)
    zh = PL.reconstruct(pp, changed)
    rr = pq1.z - zh
    pv = rr @ pp.g.T
    rep = parity.compare_quantize_polar(pp, pq1, tq.pack_codes(sl, 2), tq.pack_bits(pv.astype(np.float32) > 0),
                                        pq1.norms.astype(np.float32),
                                        np.sqrt(np.sum(rr * rr, axis=1)).astype(np.float32))
    assert rep.code_mismatch == 1 and rep.code_bad == 0 and rep.sign_mismatch == 0 and rep.cascade_keys == 1
