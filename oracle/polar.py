"""Recursive polar-angle stage 1 (the PolarQuant variant), oracle side.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages describe stage 1 as a change to polar coordinates: after the
random rotation, a vector becomes one length and a list of angles, the length
kept at high precision and each angle stored in 2 or 3 bits ("TurboQuant
tutorial", section on turning Cartesian into polar coordinates: for d = 4096
one norm and 4095 angles); the angles come from a recursive polar transform
and, after the rotation, follow a concentrated law of known analytic form, so
their quantizer needs no per-block scale ("TurboQuant deep review", section
on the breakthrough, recursive polar algorithm).  For unit vectors only the
angles carry information and the length is 1 ("Why KV-cache compression
works", section 3.3).  The pages do not spell the recursion out; the reading
taken here (d a power of two, levels l = 1 .. log2 d):

* level 1 pairs the rotated coordinates (z_{2i}, z_{2i+1}): radius
  rho_i = sqrt(z_{2i}^2 + z_{2i+1}^2) and angle psi_i = atan2(z_{2i+1}, z_{2i})
  in [0, 2 pi);
* level l >= 2 pairs the radii of level l - 1 (a, b): radius sqrt(a^2 + b^2)
  and angle atan2(b, a) in [0, pi/2];
* after log2 d levels one radius is left: ||z|| (= 1 for a unit key) and
  d/2 + d/4 + ... + 1 = d - 1 angles.

Angle laws for z uniform on the sphere (equivalently a Gaussian direction):
level-1 angles are uniform on [0, 2 pi); a level-l angle compares the norms
of two independent m = 2^(l-1)-dimensional Gaussian blocks, so sin^2 psi ~
Beta(m/2, m/2) and psi has density proportional to sin^(m-1) psi cos^(m-1) psi
= (sin 2 psi / 2)^(m-1) on [0, pi/2], symmetric about pi/4.  With
phi = psi - pi/4 the density is proportional to cos^(m-1)(2 phi) on
[-pi/4, pi/4], and s = sin(2 phi) follows the law of one coordinate of a
uniform unit vector in R^(m+1) (so cell masses are incomplete beta values).

Codebooks (2^B levels per angle, B = bits - 1 as for the scalar stage):
level 1 is the uniform quantizer of the circle (cell k = [k, k+1) 2 pi / L,
level (k + 1/2) 2 pi / L: optimal for a uniform law); level l >= 2 is the
Lloyd-Max quantizer of the phi law above, shifted by pi/4.  Levels are
rounded to float32, thresholds are the float32 midpoints (as for the scalar
codebook), and an angle's code is #{t <= fp32(psi)} (level 1: the cell of
fp32(psi)).

Reconstruction runs the recursion backwards from radius 1 with the level
values: radii of level l - 1 are (R cos c, R sin c), the last level gives
z_hat.  The QJL stage, the asymmetric score and the reconstructions then
use z_hat exactly where the scalar stage uses c[idx]: r = z - z_hat,
rho = ||r||, beta = [G r > 0], score = n (<Pi q, z_hat> + rho sqrt(pi/2)/d
<G Pi q, 2 beta - 1>), k_hat = n Pi^T z_hat.

Code layout: the d - 1 angle codes in level order (level 1's d/2 angles,
then level 2's d/4, ..., the top angle) occupy slots 0 .. d-2 of the usual
bit planes (slot d - 1 holds 0), i.e. ``tq.pack_codes`` of the slot array.
"""
from dataclasses import dataclass

import numpy as np
from scipy import integrate

from . import params as P
from . import tq

TWO_PI = 2.0 * np.pi


def levels_count(d):
    """Number of recursion levels (d a power of two, d >= 2)."""
    assert d >= 2 and d & (d - 1) == 0, "the polar recursion needs d a power of two"
    return int(np.log2(d))


def decompose(z):
    """(angles per level, top radius) of the rows of z (n, d): level 1
    angles in [0, 2 pi), higher levels in [0, pi/2]."""
    z = np.asarray(z, dtype=np.float64)
    angles = [np.mod(np.arctan2(z[:, 1::2], z[:, 0::2]), TWO_PI)]
    r = np.hypot(z[:, 0::2], z[:, 1::2])
    while r.shape[1] > 1:
        angles.append(np.arctan2(r[:, 1::2], r[:, 0::2]))
        r = np.hypot(r[:, 0::2], r[:, 1::2])
    return angles, r[:, 0]


def compose(angles, radius):
    """Inverse of ``decompose``: rows of z from per-level angles and radii."""
    r = np.asarray(radius, dtype=np.float64)[:, None]
    for a in reversed(angles[1:]):
        a = np.asarray(a, dtype=np.float64)
        nxt = np.empty((r.shape[0], 2 * r.shape[1]))
        nxt[:, 0::2] = r * np.cos(a)
        nxt[:, 1::2] = r * np.sin(a)
        r = nxt
    a = np.asarray(angles[0], dtype=np.float64)
    z = np.empty((r.shape[0], 2 * r.shape[1]))
    z[:, 0::2] = r * np.cos(a)
    z[:, 1::2] = r * np.sin(a)
    return z


# ---------------------------------------------------------------------------
# angle laws and codebooks
# ---------------------------------------------------------------------------

def angle_pdf(psi, m):
    """Density of a level angle comparing two m-dimensional Gaussian blocks
    (m = 2^(l-1)) on [0, pi/2]: sin^2 psi ~ Beta(m/2, m/2)."""
    psi = np.asarray(psi, dtype=np.float64)
    # sin^(m-1) cos^(m-1) = (sin 2psi / 2)^(m-1); normaliser from the Beta law
    from scipy import special
    logc = np.log(2.0) - special.betaln(m / 2.0, m / 2.0)
    s, c = np.sin(psi), np.cos(psi)
    with np.errstate(divide="ignore"):
        return np.exp(logc + (m - 1) * (np.log(np.clip(s, 1e-300, None)) + np.log(np.clip(c, 1e-300, None))))


def angle_cdf(psi, m):
    """CDF of that law: I_{sin^2 psi}(m/2, m/2)."""
    from scipy import special
    psi = np.clip(np.asarray(psi, dtype=np.float64), 0.0, np.pi / 2)
    return special.betainc(m / 2.0, m / 2.0, np.sin(psi) ** 2)


def _phi_mass(a, b, m):
    """Mass of [a, b] (phi = psi - pi/4 units, within [-pi/4, pi/4]): with
    s = sin 2 phi the law is the unit-sphere marginal in R^(m+1)."""
    a = np.clip(np.asarray(a, dtype=np.float64), -np.pi / 4, np.pi / 4)
    b = np.clip(np.asarray(b, dtype=np.float64), -np.pi / 4, np.pi / 4)
    return P.sphere_marginal_mass(np.sin(2 * a), np.sin(2 * b), m + 1)


def _phi_moment(a, b, m):
    """First moment of phi over [a, b] under the law, by adaptive quadrature
    of phi times the density (independent of the mass formula)."""
    a = np.atleast_1d(np.asarray(a, dtype=np.float64))
    b = np.atleast_1d(np.asarray(b, dtype=np.float64))
    out = np.empty(a.shape)
    for i in range(a.size):
        f = lambda x: x * angle_pdf(x + np.pi / 4, m)
        out[i] = integrate.quad(f, a[i], b[i], epsabs=0.0, epsrel=1e-13, limit=400)[0]
    return out


def level_codebook_fp64(m, levels):
    """Lloyd-Max levels (float64, ascending, in psi units) for the level
    angle law with blocks of dimension m."""
    sd = 0.5 / np.sqrt(m)     # phi is about N(0, 1/(4m)) for large m
    init = np.clip(P.gaussian_codebook_fp64(levels)[0] * sd, -np.pi / 4 * 0.999, np.pi / 4 * 0.999)
    c, _ = P.lloyd_max(lambda a, b: _phi_mass(a, b, m), lambda a, b: _phi_moment(a, b, m), levels, init,
                       -np.pi / 4, np.pi / 4, rel_tol=2.0 ** -40)
    return c + np.pi / 4


@dataclass
class PolarParams:
    """Rotation, projection, and per-level angle codebooks (float32 values
    held in float64)."""
    d: int
    bits: int
    code_bits: int
    pi: np.ndarray
    g: np.ndarray
    centroids: list      # per level: ascending float32 levels (level 0 = recursion level 1)
    thresholds: list     # per level: float32 midpoints (level 0: cell edges k 2pi/L, k = 1..L-1)


def init_polar(d, bits, seed):
    """Polar handle for (d, bits, seed): tq_init's rotation and projection,
    per-level angle codebooks of 2^(bits-1) levels."""
    base = P.init(d, bits, seed)
    B = bits - 1
    L = 1 << B
    nl = levels_count(d)
    cents, thr = [], []
    # level 1: uniform quantizer of the circle
    c1 = ((np.arange(L) + 0.5) * TWO_PI / L).astype(np.float32).astype(np.float64)
    t1 = (np.arange(1, L) * TWO_PI / L).astype(np.float32).astype(np.float64)
    cents.append(c1)
    thr.append(t1)
    for lvl in range(2, nl + 1):
        m = 1 << (lvl - 1)
        c = level_codebook_fp64(m, L).astype(np.float32).astype(np.float64)
        t = P.thresholds_from_centroids(c)
        cents.append(c)
        thr.append(t)
    return PolarParams(d, bits, B, base.pi, base.g, cents, thr)


# ---------------------------------------------------------------------------
# quantize, reconstruct, score
# ---------------------------------------------------------------------------

def quantize_angles(pp: PolarParams, angles):
    """Per-level codes #{t <= fp32(angle)} (level 1: its uniform cell)."""
    out = []
    for lvl, a in enumerate(angles):
        a32 = np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)
        out.append(np.searchsorted(pp.thresholds[lvl], a32, side="right").astype(np.int64))
    return out


def reconstruct(pp: PolarParams, codes):
    """z_hat rows from per-level codes, radius 1."""
    angles = [pp.centroids[lvl][c] for lvl, c in enumerate(codes)]
    n = codes[0].shape[0]
    return compose(angles, np.ones(n))


def slots(codes):
    """Per-level codes -> (n, d) slot array (level order, slot d-1 = 0)."""
    n = codes[0].shape[0]
    flat = np.concatenate(codes, axis=1)
    return np.concatenate([flat, np.zeros((n, 1), dtype=np.int64)], axis=1)


def unslot(slot_idx, d):
    """(n, d) slot array -> per-level codes."""
    out, at, k = [], 0, d // 2
    while k >= 1:
        out.append(np.asarray(slot_idx[:, at:at + k], dtype=np.int64))
        at += k
        k //= 2
    return out


@dataclass
class PolarQuantized:
    codes: list          # per level (n, d / 2^l)
    angles: list         # per level, float64 (pre-quantization values)
    beta: np.ndarray     # (n, d) QJL sign bits
    norms: np.ndarray
    rnorms: np.ndarray
    z: np.ndarray
    zhat: np.ndarray
    p: np.ndarray


def quantize(pp: PolarParams, keys):
    """Normalize, rotate, polar-decompose, quantize the angles, then the QJL
    stage on r = z - z_hat (as ``tq.quantize`` with z_hat for c[idx])."""
    keys = np.asarray(keys, dtype=np.float64)
    norms, u = tq.normalize(keys)
    z = u @ pp.pi.T
    angles, _ = decompose(z)
    codes = quantize_angles(pp, angles)
    zhat = reconstruct(pp, codes)
    r = z - zhat
    rn = np.sqrt(np.sum(r * r, axis=1))
    p = r @ pp.g.T
    beta = p.astype(np.float32) > 0
    return PolarQuantized(codes, angles, beta, norms, rn, z, zhat, p)


def scores(pp: PolarParams, queries, codes, beta, norms, rnorms):
    """(m, n) asymmetric scores of queries against polar-coded keys."""
    q = np.asarray(queries, dtype=np.float64)
    v = q @ pp.pi.T
    w = v @ pp.g.T
    zhat = reconstruct(pp, codes)
    sg = np.where(np.asarray(beta), 1.0, -1.0)
    scale = np.asarray(rnorms, dtype=np.float64) * tq.QJL_CONST / pp.d
    return np.asarray(norms, dtype=np.float64)[None, :] * (v @ zhat.T + scale[None, :] * (w @ sg.T))


def dequant(pp: PolarParams, codes, norms):
    """Stage-1 reconstruction n Pi^T z_hat."""
    return np.asarray(norms, dtype=np.float64)[:, None] * (reconstruct(pp, codes) @ pp.pi)
