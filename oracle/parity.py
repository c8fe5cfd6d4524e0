"""Comparison rules between the library's outputs and the oracle's.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Rules (all derived from the float32 arithmetic of the library against the
float64 oracle; the window and the rate come with the method's statement of
parity):

* codes: bit-exact, except that an index may differ where the oracle's
  rotated coordinate z_j lies within 1e-6 of a threshold.  Such mismatches
  are counted and must stay below 1e-5 of all coordinates.
* signs: bit-exact, except where the oracle's projected residual lies within
  1e-6 of zero in JL-normalised units, |p_j| / sqrt(d) < 1e-6.  (sign(p) does
  not depend on the scale of the projection; with the JL normalisation
  S / sqrt(d) the projected value has the same scale as a rotated
  coordinate, so the window means the same for both decisions.)  A key whose
  code changed inside the window has a different residual, so its signs
  and rho are not compared; such keys are counted.
* norms: |n_gpu - n| <= d 2^-24 n (float32 sum of d squares, worst case).
* rnorms: |rho_gpu - rho| <= sqrt(d) 1e-6 + d 2^-24 rho.
* scores: |s_gpu - s| <= 1e-3 ||q|| n_k per score.
* stage-1 reconstruction: ||k_hat_gpu - k_hat|| <= 1e-5 ||k_hat|| per key.
* padding bits past d are zero.
* top-k per query: the k indices are distinct and in range, and the scores
  come best first (ties in ascending index).  Each returned score is within
  the score tolerance of the oracle's score for that key.  The set may
  differ from the oracle's only near the k-th score: a returned key's oracle
  score is at least the oracle's k-th score minus twice the row's largest
  score tolerance, and every key whose oracle score exceeds the k-th by more
  than that is returned.
"""
from dataclasses import dataclass, field

import numpy as np

from . import tq

CODE_WINDOW = 1e-6
SIGN_WINDOW = 1e-6
MISMATCH_RATE = 1e-5
SCORE_TOL = 1e-3
DEQUANT_TOL = 1e-5


@dataclass
class QuantizeReport:
    elements: int = 0
    code_mismatch: int = 0
    code_bad: int = 0
    sign_mismatch: int = 0
    sign_bad: int = 0
    cascade_keys: int = 0
    norm_bad: int = 0
    rnorm_bad: int = 0
    padding_bad: int = 0
    worst: dict = field(default_factory=dict)

    @property
    def mismatch_rate(self):
        return (self.code_mismatch + self.sign_mismatch) / max(self.elements, 1)

    def ok(self):
        return (self.code_bad == 0 and self.sign_bad == 0 and self.norm_bad == 0 and self.rnorm_bad == 0
                and self.padding_bad == 0 and self.mismatch_rate < MISMATCH_RATE)

    def cascade(self):
        return self.cascade_keys


def _padding_zero(words, d):
    extra = words.shape[-1] * 32 - d
    if extra == 0:
        return 0
    mask = np.uint32(((1 << extra) - 1) << (32 - extra))
    return int(np.count_nonzero(words[..., -1].astype(np.uint32) & mask))


def compare_quantize(params, qz, codes, signs, norms, rnorms):
    """qz: oracle ``tq.Quantized``; the rest: library outputs as numpy."""
    d = params.d
    codes = np.asarray(codes).view(np.uint32)
    signs = np.asarray(signs).view(np.uint32)
    norms = np.asarray(norms, dtype=np.float64)
    rnorms = np.asarray(rnorms, dtype=np.float64)
    rep = QuantizeReport(elements=2 * qz.idx.size)
    if params.hi:
        # fractional widths: B full planes, then the plane of the first hi
        # coordinates; the decision window is each coordinate's own set
        n, b, w = codes.shape[0], params.code_bits, tq.words_per_plane(d)
        codes = codes.reshape(n, -1)
        rep.padding_bad = (_padding_zero(codes[:, :b * w].reshape(n, b, w), d) + _padding_zero(codes[:, b * w:], params.hi)
                           + _padding_zero(signs, d))
        idx = tq.unpack_codes_split(codes, d, b, params.hi)
        h = params.hi
        dist = np.concatenate(
            [np.min(np.abs(qz.z[:, :h, None] - params.thresholds_hi[None, None, :]), axis=2),
             np.min(np.abs(qz.z[:, h:, None] - params.thresholds[None, None, :]), axis=2)], axis=1)
    else:
        rep.padding_bad = _padding_zero(codes, d) + _padding_zero(signs, d)
        idx = tq.unpack_codes(codes, d)
        dist = np.min(np.abs(qz.z[:, :, None] - params.thresholds[None, None, :]), axis=2) \
            if len(params.thresholds) else np.full(qz.z.shape, np.inf)
    cmis = idx != qz.idx
    rep.code_mismatch = int(cmis.sum())
    rep.code_bad = int((cmis & (dist >= CODE_WINDOW)).sum())
    flipped = cmis.any(axis=1)
    rep.cascade_keys = int(flipped.sum())

    beta = tq.unpack_bits(signs, d)
    keep = ~flipped
    smis = (beta != qz.beta) & keep[:, None]
    pn = np.abs(qz.p) / np.sqrt(d)
    rep.sign_mismatch = int(smis.sum())
    rep.sign_bad = int((smis & (pn >= SIGN_WINDOW)).sum())

    ntol = d * 2.0 ** -24 * qz.norms
    rep.norm_bad = int((np.abs(norms - qz.norms) > ntol).sum())
    rtol = np.sqrt(d) * 1e-6 + d * 2.0 ** -24 * qz.rnorms
    rep.rnorm_bad = int(((np.abs(rnorms - qz.rnorms) > rtol) & keep).sum())
    if rep.code_bad:
        i = np.argwhere(cmis & (dist >= CODE_WINDOW))[0]
        rep.worst["code"] = (tuple(int(x) for x in i), float(dist[tuple(i)]))
    if rep.sign_bad:
        i = np.argwhere(smis & (pn >= SIGN_WINDOW))[0]
        rep.worst["sign"] = (tuple(int(x) for x in i), float(pn[tuple(i)]))
    return rep


def score_violations(s_gpu, s_ref, queries, norms, keep=None):
    """Count of scores outside 1e-3 ||q|| n_k; s arrays are (m, n)."""
    s_gpu = np.asarray(s_gpu, dtype=np.float64)
    s_ref = np.asarray(s_ref, dtype=np.float64)
    qn = np.linalg.norm(np.asarray(queries, dtype=np.float64), axis=1)
    tol = SCORE_TOL * qn[:, None] * np.asarray(norms, dtype=np.float64)[None, :]
    bad = np.abs(s_gpu - s_ref) > tol
    if keep is not None:
        bad &= np.asarray(keep)[None, :]
    ratio = np.abs(s_gpu - s_ref) / np.maximum(tol, 1e-300)
    if keep is not None:
        ratio = ratio[:, np.asarray(keep)]
    return int(bad.sum()), float(ratio.max()) if ratio.size else 0.0


def dequant_violations(k_gpu, k_ref):
    k_gpu = np.asarray(k_gpu, dtype=np.float64)
    k_ref = np.asarray(k_ref, dtype=np.float64)
    err = np.linalg.norm(k_gpu - k_ref, axis=1)
    ref = np.linalg.norm(k_ref, axis=1)
    bad = err > DEQUANT_TOL * ref
    ratio = err / np.maximum(DEQUANT_TOL * ref, 1e-300)
    return int(bad.sum()), float(ratio.max()) if ratio.size else 0.0


@dataclass
class TopkReport:
    rows: int = 0
    swapped: int = 0        # keys in one set and not the other (both near the k-th score)
    bad: list = field(default_factory=list)

    def ok(self):
        return not self.bad


def compare_topk(idx_gpu, s_gpu, s_ref, queries, norms, k):
    """Check (m, k') GPU top-k lists against the oracle's (m, n) scores."""
    idx_gpu = np.asarray(idx_gpu, dtype=np.int64)
    s_gpu = np.asarray(s_gpu, dtype=np.float64)
    s_ref = np.asarray(s_ref, dtype=np.float64)
    m, n = s_ref.shape
    kk = min(int(k), n)
    norms = np.asarray(norms, dtype=np.float64)
    qn = np.linalg.norm(np.asarray(queries, dtype=np.float64), axis=1)
    rep = TopkReport(rows=m)
    ref_idx, ref_s = tq.topk(s_ref, kk)
    for i in range(m):
        ids, vals = idx_gpu[i, :kk], s_gpu[i, :kk]
        tol = SCORE_TOL * qn[i] * norms
        if len(set(ids.tolist())) != kk or ids.min() < 0 or ids.max() >= n:
            rep.bad.append((i, "indices not distinct or out of range"))
            continue
        order_ok = all(vals[j] > vals[j + 1] or (vals[j] == vals[j + 1] and ids[j] < ids[j + 1])
                       for j in range(kk - 1))
        if not order_ok:
            rep.bad.append((i, "not best first"))
        if np.any(np.abs(vals - s_ref[i, ids]) > tol[ids]):
            rep.bad.append((i, "returned score off"))
        kth = ref_s[i, -1]
        slack = 2.0 * tol.max()
        if np.any(s_ref[i, ids] < kth - slack):
            rep.bad.append((i, "returned key well below the k-th score"))
        must = np.nonzero(s_ref[i] > kth + slack)[0]
        if not set(must.tolist()) <= set(ids.tolist()):
            rep.bad.append((i, "missed a key well above the k-th score"))
        rep.swapped += len(set(ids.tolist()) ^ set(ref_idx[i].tolist())) // 2
    return rep
