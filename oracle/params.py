"""Method parameters: rotation Pi, projection G and the scalar codebook.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

* Rotation.  "TurboQuant deep review" (freelamp.com), breakthrough section,
  and "TurboQuant digest" (juejin.cn), section 2: vectors are first multiplied
  by a random orthogonal matrix so that their coordinates follow a
  concentrated, predictable law.  Reading: Pi is Haar distributed, obtained
  from the QR factorisation of a seeded d x d standard-normal matrix with the
  signs of R's diagonal moved into Q (Mezzadri, "How to generate random
  matrices from the classical compact groups", Notices AMS 2007).  It is
  rounded to float32, the precision the library stores.
* Projection.  "TurboQuant tutorial" (gitcode.csdn.net), QJL section: the
  residual goes through a Gaussian JL matrix whose output has as many
  dimensions as the input.  Reading: the residual lives in rotated
  coordinates, so the projection of the original-domain residual is
  S = G Pi with G a seeded d x d matrix of iid N(0, 1) entries (S is again
  iid Gaussian because G is independent of the orthogonal Pi).  G is rounded
  to float32.
* Codebook.  "Why KV-cache compression works ..." (nonndazone.ru), section
  3.2 / 3.4, and the freelamp review: centroids sit where the probability
  mass is and are precomputed once for every token; "TurboQuant tutorial",
  QJL section: each value is replaced by the nearest allowed value.  Reading:
  the allowed values are the Lloyd-Max (minimum mean-square error) quantizer
  with 2**B levels for the exact law of one coordinate of a uniformly random
  unit vector in R^d,

      f_d(z) = Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)) * (1 - z^2)^((d-3)/2),

  on [-1, 1]; its CDF is the regularised incomplete beta function
  I_{(1+z)/2}((d-1)/2, (d-1)/2) and its first moment has the closed form
  int z f_d = -C (1 - z^2)^((d-1)/2) / (d - 1).  Centroids are rounded to
  float32; decision thresholds are the float32 midpoints of adjacent float32
  centroids.
* Bit split.  "TurboQuant tutorial", section on the method: a 2-bit coarse
  stage gives 3 bits in total and a 3-bit stage 4 bits, one of them the QJL
  sign.  So B = bits - 1 codebook bits.
"""
from dataclasses import dataclass

import numpy as np
from scipy import special

from . import rng

STREAM_ROTATION = 0
STREAM_PROJECTION = 1


def haar_rotation(d, seed):
    """Haar-random orthogonal d x d matrix (float64) from the rotation stream."""
    a = rng.normals(seed, STREAM_ROTATION, d * d).reshape(d, d)
    q, r = np.linalg.qr(a)
    signs = np.sign(np.diag(r))
    signs[signs == 0] = 1.0
    return q * signs[None, :]


def gaussian_projection(d, seed):
    """d x d matrix of iid N(0, 1) draws (float64) from the projection stream."""
    return rng.normals(seed, STREAM_PROJECTION, d * d).reshape(d, d)


def projection_matrix(d, seed):
    """The QJL matrix G of a seeded handle: the projection stream's N(0, 1)
    draws rounded once to float16 precision (11 significant bits, nearest
    even), as float64.  The pages ask for iid standard normal entries and
    fix no storage precision; entries with 11 significant bits are exact
    operands for float16 matrix arithmetic, and the rounding moves each
    entry by at most 2^-11 of itself."""
    return gaussian_projection(d, seed).astype(np.float16).astype(np.float64)


# ----------------------------------------------------------------------------
# Lloyd-Max on a density given by its cell mass and cell first moment.
# ----------------------------------------------------------------------------

def lloyd_max(mass, moment, levels, init, lo, hi, rel_tol=2.0 ** -46, settle=20,
              max_iter=200000):
    """Lloyd-Max fixed point: thresholds at midpoints, centroids at cell means.

    ``mass(a, b)`` and ``moment(a, b)`` return the probability and the first
    moment of the interval(s) [a, b]; ``lo`` / ``hi`` bound the support.  The
    level set is kept symmetric about zero (every density used here is even).
    Iteration stops ``settle`` steps after the largest centroid move first
    drops below ``rel_tol`` times the largest centroid (the float64 noise
    floor of the cell integrals is a few 1e-15 relative).
    Returns (centroids, iterations).
    """
    c = np.array(init, dtype=np.float64)
    assert c.shape == (levels,)
    remaining = None
    near = 0
    for it in range(1, max_iter + 1):
        t = np.concatenate(([lo], 0.5 * (c[:-1] + c[1:]), [hi]))
        new = moment(t[:-1], t[1:]) / mass(t[:-1], t[1:])
        new = 0.5 * (new - new[::-1])
        delta = np.max(np.abs(new - c)) / np.max(np.abs(new))
        c = new
        if remaining is None and delta <= rel_tol:
            remaining = settle
        # at the float64 noise floor the move jitters around ~1e-14 and never
        # settles below rel_tol: accept after a long stretch near it
        near = near + 1 if delta <= 1e-11 else 0
        if near >= 300:
            return c, it
        if remaining is not None:
            remaining -= 1
            if remaining <= 0:
                return c, it
    raise RuntimeError("Lloyd-Max did not converge")


def sphere_marginal_constant(d):
    """Normaliser Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)) of f_d."""
    return np.exp(special.gammaln(d / 2.0) - special.gammaln((d - 1) / 2.0)) / np.sqrt(np.pi)


def sphere_marginal_pdf(z, d):
    z = np.asarray(z, dtype=np.float64)
    return sphere_marginal_constant(d) * np.power(np.clip(1.0 - z * z, 0.0, None), (d - 3) / 2.0)


def sphere_marginal_cdf(z, d):
    a = (d - 1) / 2.0
    return special.betainc(a, a, np.clip((1.0 + np.asarray(z, dtype=np.float64)) / 2.0, 0.0, 1.0))


def sphere_marginal_sf(z, d):
    """1 - CDF, computed directly (no cancellation in the upper tail)."""
    a = (d - 1) / 2.0
    return special.betainc(a, a, np.clip((1.0 - np.asarray(z, dtype=np.float64)) / 2.0, 0.0, 1.0))


def sphere_marginal_mass(a, b, d):
    """P(a < z < b); upper-half cells use the survival function."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    lower = sphere_marginal_cdf(b, d) - sphere_marginal_cdf(a, d)
    upper = sphere_marginal_sf(a, d) - sphere_marginal_sf(b, d)
    return np.where(a >= 0.0, upper, lower)


def sphere_marginal_moment(a, b, d):
    """int_a^b z f_d(z) dz from the closed-form antiderivative."""
    c = sphere_marginal_constant(d)
    e = (d - 1) / 2.0

    def anti(z):
        # (1 - z^2)^e as exp(e * log1p(-z^2)): keeps full relative precision
        # when e = (d-1)/2 is large
        z2 = np.minimum(np.asarray(z, dtype=np.float64) ** 2, 1.0)
        with np.errstate(divide="ignore"):
            return -c * np.exp(e * np.log1p(-z2)) / (d - 1)

    return anti(b) - anti(a)


def sphere_codebook_fp64(d, levels):
    """Lloyd-Max levels for f_d in float64 (ascending, symmetric)."""
    if levels == 1:
        return np.zeros(1), 0
    # initial levels: quantile midpoints of the large-d normal limit N(0, 1/d)
    from scipy.stats import norm
    p = (np.arange(levels) + 0.5) / levels
    init = norm.ppf(p) / np.sqrt(d)
    init = np.clip(init, -0.999, 0.999)
    return lloyd_max(lambda a, b: sphere_marginal_mass(a, b, d),
                     lambda a, b: sphere_marginal_moment(a, b, d),
                     levels, init, -1.0, 1.0)


def gaussian_codebook_fp64(levels):
    """Lloyd-Max levels for N(0, 1) (the textbook case, used as a pin)."""
    from scipy.stats import norm
    p = (np.arange(levels) + 0.5) / levels
    init = norm.ppf(p)

    def mass(a, b):
        return np.where(np.asarray(a) >= 0.0, norm.sf(a) - norm.sf(b), norm.cdf(b) - norm.cdf(a))

    def moment(a, b):
        return norm.pdf(a) - norm.pdf(b)

    return lloyd_max(mass, moment, levels, init, -np.inf, np.inf)


def codebook_mse(centroids, d):
    """Per-coordinate MSE of the level set under f_d (quadrature-free form).

    E[(z - c(z))^2] = E[z^2] - sum_i c_i (2 m1_i - c_i m0_i); E[z^2] = 1/d.
    """
    c = np.asarray(centroids, dtype=np.float64)
    t = np.concatenate(([-1.0], 0.5 * (c[:-1] + c[1:]), [1.0]))
    m0 = sphere_marginal_mass(t[:-1], t[1:], d)
    m1 = sphere_marginal_moment(t[:-1], t[1:], d)
    return 1.0 / d - np.sum(c * (2.0 * m1 - c * m0))


@dataclass
class Params:
    """Everything ``init(d, bits, seed)`` produces.

    ``pi`` and ``g`` hold the float32-rounded matrices as float64 arrays;
    ``centroids`` the float32-rounded levels (ascending, float64 array);
    ``thresholds`` the float32 midpoints between adjacent levels.
    """
    d: int
    bits: int
    seed: int
    pi: np.ndarray
    g: np.ndarray
    centroids: np.ndarray
    thresholds: np.ndarray
    # fractional widths: rotated coordinates 0 .. hi-1 use the finer level
    # set below (one more index bit); hi = 0 for a plain handle
    hi: int = 0
    centroids_hi: np.ndarray = None
    thresholds_hi: np.ndarray = None

    @property
    def code_bits(self):
        return self.bits - 1

    @property
    def levels(self):
        return 1 << (self.bits - 1)


def thresholds_from_centroids(c32):
    """float32 midpoints of adjacent float32 centroids (exact sum in float64)."""
    c = np.asarray(c32, dtype=np.float64)
    return (0.5 * (c[:-1] + c[1:])).astype(np.float32).astype(np.float64)


def init(d, bits, seed):
    """Build the method's parameters for (d, bits, seed).  bits = B + 1."""
    if not (2 <= d <= 4096):
        raise ValueError("d must lie in [2, 4096]")
    if not (2 <= bits <= 5):
        raise ValueError("bits must lie in [2, 5]")
    levels = 1 << (bits - 1)
    pi = haar_rotation(d, seed).astype(np.float32).astype(np.float64)
    g = projection_matrix(d, seed)
    c64, _ = sphere_codebook_fp64(d, levels)
    c32 = c64.astype(np.float32).astype(np.float64)
    return Params(d, bits, int(seed), pi, g, c32, thresholds_from_centroids(c32))


def init_split(d, bits, hi, seed):
    """Fractional widths: ``init(d, bits, seed)`` plus a second Lloyd-Max
    level set with twice the levels (one more index bit) for the rotated
    coordinates 0 .. hi-1.  The stage-1 budget is then (bits - 1) + hi / d
    bits per coordinate, bits + hi / d with the QJL sign bit; e.g. d = 128,
    hi = 64 gives 2.5 bits from bits = 2 and 3.5 from bits = 3.  Every
    rotated coordinate has the same law, so which coordinates get the finer
    set does not change the expected error; the first hi keeps the layout
    simple.  bits in [2, 4] (the finer set stays within 16 levels)."""
    if not (2 <= bits <= 4):
        raise ValueError("bits must lie in [2, 4] for fractional widths")
    if not (0 <= hi <= d):
        raise ValueError("hi must lie in [0, d]")
    pr = init(d, bits, seed)
    c64, _ = sphere_codebook_fp64(d, 1 << bits)
    c32 = c64.astype(np.float32).astype(np.float64)
    pr.hi = int(hi)
    pr.centroids_hi = c32
    pr.thresholds_hi = thresholds_from_centroids(c32)
    return pr


def hadamard_rotation(d, seed):
    """Randomized Hadamard rotation H diag(sigma) / sqrt(d) (float64 of the
    float32 entries): H the Sylvester Hadamard matrix (scipy), sigma the
    stream-2 signs.  The tutorial page's 4-D example rotates with H_4 / 2.
    d must be a power of two."""
    if d < 2 or d > 4096 or d & (d - 1):
        raise ValueError("d must be a power of two in [2, 4096]")
    from scipy.linalg import hadamard
    sigma = rng.signs(seed, 2, d)
    scale = np.float32(1.0 / np.sqrt(d))
    return (hadamard(d).astype(np.float64) * sigma[None, :] * np.float64(scale)).astype(np.float32).astype(np.float64)


def init_hadamard(d, bits, seed):
    """Parameters with the randomized Hadamard rotation; G and the codebook
    as in ``init``."""
    if not (2 <= bits <= 5):
        raise ValueError("bits must lie in [2, 5]")
    levels = 1 << (bits - 1)
    pi = hadamard_rotation(d, seed)
    g = projection_matrix(d, seed)
    c64, _ = sphere_codebook_fp64(d, levels)
    c32 = c64.astype(np.float32).astype(np.float64)
    return Params(d, bits, int(seed), pi, g, c32, thresholds_from_centroids(c32))


def explicit(d, bits, pi, g):
    """Parameters with given matrices (codebook still from ``d`` and ``bits``)."""
    levels = 1 << (bits - 1)
    c64, _ = sphere_codebook_fp64(d, levels)
    c32 = c64.astype(np.float32).astype(np.float64)
    return Params(d, bits, -1,
                  np.asarray(pi, dtype=np.float32).astype(np.float64),
                  np.asarray(g, dtype=np.float32).astype(np.float64),
                  c32, thresholds_from_centroids(c32))
