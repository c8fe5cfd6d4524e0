"""Comparison rules between the library's outputs and the oracle's.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Rules (all derived from the float32 arithmetic of the library against the
float64 oracle; the window and the rate come with the method's statement of
parity):

* codes: bit-exact, except that an index may differ where the oracle's
  rotated coordinate z_j lies within 1e-6 of a threshold.  Such mismatches
  are counted and must stay below 1e-5 of all coordinates.
* signs: bit-exact, except where the reference projection p_j = (G r)_j
  lies within 1e-6 of zero (the decision boundary of the QJL bit).  For a
  key whose code changed inside the window the reference is the oracle run
  on the library's own codes: r = z - c[idx_gpu], rho = ||r||, p = G r
  (a changed code changes the residual, and so rho and many signs of that
  key).  Such keys are counted, and their signs and rho are compared with
  that recomputed reference, not skipped.  The count of sign mismatches
  outside the wider window |p_j| / sqrt(d) < 1e-6 (the projection with the
  Johnson-Lindenstrauss normalisation S / sqrt(d), on the scale of a
  rotated coordinate) is reported beside it.
* norms: |n_gpu - n| <= d 2^-24 n (float32 sum of d squares, worst case).
* rnorms: |rho_gpu - rho| <= sqrt(d) 1e-6 + d 2^-24 rho.
* scores: |s_gpu - s| <= 1e-3 ||q|| n_k per score.  End to end (the
  library's own quantizer output scored by the library), s is the oracle's
  estimator on the library's decisions (its codes and signs, each checked
  above against the oracle's own) with the oracle's n and the reference
  rho: a decision that flips inside its window moves a score by more than
  that bound (one QJL sign moves it by 2 n rho sqrt(pi/2) / d |w_j|, with
  w_j of the size of ||q||: several times 1e-3 ||q|| n at d = 128), so the
  bound holds only given the same decisions.  Keys with any flipped
  decision are counted (``decision_keys``) and scored all the same.
* stage-1 reconstruction: ||k_hat_gpu - k_hat|| <= 1e-5 ||k_hat|| per key.
* padding bits past d are zero.
* every comparison is written so that a NaN or an infinity on the
  library's side is a violation (a value passes only when its error is
  known to be within the bound).
* top-k per query: the k indices are distinct and in range, and the scores
  come best first (ties in ascending index).  Each returned score is within
  the score tolerance of the oracle's score for that key.  The set may
  differ from the oracle's only near the k-th score: a returned key's oracle
  score is at least the oracle's k-th score minus twice the row's largest
  score tolerance, and every key whose oracle score exceeds the k-th by more
  than that is returned.
"""
from dataclasses import dataclass, field, replace

import numpy as np

from . import tq

CODE_WINDOW = 1e-6
SIGN_WINDOW = 1e-6
MISMATCH_RATE = 1e-5
SCORE_TOL = 1e-3
DEQUANT_TOL = 1e-5


def _within(err, tol):
    """True where err <= tol; NaN and infinite errors are outside."""
    err = np.asarray(err, dtype=np.float64)
    return np.isfinite(err) & (err <= tol)


@dataclass
class QuantizeReport:
    elements: int = 0
    code_mismatch: int = 0
    code_bad: int = 0
    sign_mismatch: int = 0
    sign_bad: int = 0                 # outside |p| < 1e-6
    sign_bad_normalized: int = 0      # outside |p| / sqrt(d) < 1e-6 (reported only)
    cascade_keys: int = 0
    norm_bad: int = 0
    rnorm_bad: int = 0
    nonfinite: int = 0
    padding_bad: int = 0
    decision_keys: int = 0            # keys with any code or sign mismatch
    worst: dict = field(default_factory=dict)
    reference: object = field(default=None, repr=False)
    idx: object = field(default=None, repr=False)    # the library's indices, unpacked (n, d)
    beta: object = field(default=None, repr=False)   # the library's sign bits, unpacked (n, d)

    @property
    def mismatch_rate(self):
        return (self.code_mismatch + self.sign_mismatch) / max(self.elements, 1)

    def ok(self):
        return (self.code_bad == 0 and self.sign_bad == 0 and self.norm_bad == 0 and self.rnorm_bad == 0
                and self.padding_bad == 0 and self.mismatch_rate < MISMATCH_RATE)

    def cascade(self):
        return self.cascade_keys

    def summary(self):
        return {"elements": self.elements, "code_mismatch": self.code_mismatch, "sign_mismatch": self.sign_mismatch,
                "mismatch_rate": self.mismatch_rate, "code_bad": self.code_bad, "sign_bad": self.sign_bad,
                "sign_bad_normalized_window": self.sign_bad_normalized, "cascade_keys": self.cascade_keys,
                "decision_keys": self.decision_keys,
                "norm_bad": self.norm_bad, "rnorm_bad": self.rnorm_bad, "padding_bad": self.padding_bad}


def _padding_zero(words, d):
    extra = words.shape[-1] * 32 - d
    if extra == 0:
        return 0
    mask = np.uint32(((1 << extra) - 1) << (32 - extra))
    return int(np.count_nonzero(words[..., -1].astype(np.uint32) & mask))


def _threshold_distance(z, t):
    """Distance of each z to the nearest threshold of the ascending list t
    (inf when there is none)."""
    t = np.asarray(t, dtype=np.float64)
    if len(t) == 0:
        return np.full(np.shape(z), np.inf)
    i = np.searchsorted(t, z)
    below = t[np.clip(i - 1, 0, len(t) - 1)]
    above = t[np.clip(i, 0, len(t) - 1)]
    return np.minimum(np.abs(z - below), np.abs(z - above))


def reference_for_codes(params, qz, idx):
    """The oracle's quantizer output with the stage-1 indices replaced by
    ``idx`` (n, d): residual, rho, projection and signs recomputed from the
    oracle's z for the keys whose indices differ; the other keys unchanged."""
    idx = np.asarray(idx, dtype=np.int64)
    changed = (idx != qz.idx).any(axis=1)
    if not changed.any():
        return qz
    beta, p, rn = qz.beta.copy(), qz.p.copy(), qz.rnorms.copy()
    r, rn_c = tq.residual(params, qz.z[changed], idx[changed])
    p_c, beta_c = tq.project_signs(params, r)
    beta[changed], p[changed], rn[changed] = beta_c, p_c, rn_c
    return replace(qz, idx=idx.copy(), beta=beta, p=p, rnorms=rn)


def compare_quantize(params, qz, codes, signs, norms, rnorms):
    """qz: oracle ``tq.Quantized``; the rest: library outputs as numpy.
    ``report.reference`` is the oracle output on the library's codes
    (``reference_for_codes``); ``report.idx`` / ``report.beta`` are the
    library's decisions unpacked (``e2e_scores`` scores them)."""
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
        dist = np.concatenate([_threshold_distance(qz.z[:, :h], params.thresholds_hi),
                               _threshold_distance(qz.z[:, h:], params.thresholds)], axis=1)
    else:
        rep.padding_bad = _padding_zero(codes, d) + _padding_zero(signs, d)
        idx = tq.unpack_codes(codes, d)
        dist = _threshold_distance(qz.z, params.thresholds)
    cmis = idx != qz.idx
    rep.code_mismatch = int(cmis.sum())
    rep.code_bad = int((cmis & (dist >= CODE_WINDOW)).sum())
    rep.cascade_keys = int(cmis.any(axis=1).sum())

    ref = reference_for_codes(params, qz, idx)
    rep.reference = ref
    beta = tq.unpack_bits(signs, d)
    smis = beta != ref.beta
    pa = np.abs(ref.p)
    rep.sign_mismatch = int(smis.sum())
    rep.sign_bad = int((smis & (pa >= SIGN_WINDOW)).sum())
    rep.sign_bad_normalized = int((smis & (pa / np.sqrt(d) >= SIGN_WINDOW)).sum())
    rep.decision_keys = int((cmis.any(axis=1) | smis.any(axis=1)).sum())
    rep.idx, rep.beta = idx, beta

    rep.nonfinite = int((~np.isfinite(norms)).sum() + (~np.isfinite(rnorms)).sum())
    ntol = d * 2.0 ** -24 * qz.norms
    rep.norm_bad = int((~_within(np.abs(norms - qz.norms), ntol)).sum())
    rtol = np.sqrt(d) * 1e-6 + d * 2.0 ** -24 * ref.rnorms
    rep.rnorm_bad = int((~_within(np.abs(rnorms - ref.rnorms), rtol)).sum())
    if rep.code_bad:
        i = np.argwhere(cmis & (dist >= CODE_WINDOW))[0]
        rep.worst["code"] = (tuple(int(x) for x in i), float(dist[tuple(i)]))
    if rep.sign_bad:
        i = np.argwhere(smis & (pa >= SIGN_WINDOW))[0]
        rep.worst["sign"] = (tuple(int(x) for x in i), float(pa[tuple(i)]))
    return rep


def e2e_scores(params, rep, queries, norms, rows=slice(None)):
    """Reference for the library's end-to-end scores of keys ``rows``: the
    oracle's estimator on the library's codes and signs with the oracle's
    norms ``norms`` (of those keys) and the reference rho."""
    return tq.scores(params, queries, rep.idx[rows], rep.beta[rows], norms, rep.reference.rnorms[rows])


def polar_angle_distance(pp, angles):
    """(n, d) distance of every angle (slot order) to its level's nearest
    decision boundary; level 1 also counts the cut of the circle at 0 = 2 pi
    (an angle just below 2 pi and one at 0 lie in different cells); the
    unused slot d - 1 gets inf."""
    from . import polar
    out = []
    for lvl, a in enumerate(angles):
        t = np.asarray(pp.thresholds[lvl], dtype=np.float64)
        if lvl == 0:
            t = np.concatenate(([0.0], t, [polar.TWO_PI]))
        out.append(_threshold_distance(np.asarray(a, dtype=np.float64), t))
    n = out[0].shape[0]
    return np.concatenate(out + [np.full((n, 1), np.inf)], axis=1)


def compare_quantize_polar(pp, pq, codes, signs, norms, rnorms):
    """The quantize rules for a polar handle (``oracle.polar``): angle codes
    (slot order in the bit planes) bit-exact except where the angle lies
    within 1e-6 of a decision boundary of its level; signs, norms and rho as
    in ``compare_quantize``, keys with a changed code compared with the
    oracle recomputed from the library's codes (z_hat, r, rho, p).
    ``report.reference`` holds that reference (codes, beta, p, rnorms)."""
    from . import polar
    d = pp.d
    codes = np.asarray(codes).view(np.uint32)
    signs = np.asarray(signs).view(np.uint32)
    norms = np.asarray(norms, dtype=np.float64)
    rnorms = np.asarray(rnorms, dtype=np.float64)
    rep = QuantizeReport(elements=2 * pq.z.size)
    slots = tq.unpack_codes(codes, d)
    rep.padding_bad = _padding_zero(codes, d) + _padding_zero(signs, d) + int(np.count_nonzero(slots[:, d - 1]))
    ref_slots = polar.slots(pq.codes)
    dist = polar_angle_distance(pp, pq.angles)
    cmis = slots != ref_slots
    rep.code_mismatch = int(cmis.sum())
    rep.code_bad = int((cmis & (dist >= CODE_WINDOW)).sum())
    changed = cmis.any(axis=1)
    rep.cascade_keys = int(changed.sum())
    beta, p, rn = pq.beta.copy(), pq.p.copy(), pq.rnorms.copy()
    lib_codes = polar.unslot(slots, d)
    if changed.any():
        zh = polar.reconstruct(pp, [c[changed] for c in lib_codes])
        r = pq.z[changed] - zh
        rn[changed] = np.sqrt(np.sum(r * r, axis=1))
        p[changed] = r @ pp.g.T
        beta[changed] = p[changed].astype(np.float32) > 0
    ref = dict(codes=lib_codes, beta=beta, p=p, rnorms=rn)
    rep.reference = ref
    lib_beta = tq.unpack_bits(signs, d)
    smis = lib_beta != beta
    pa = np.abs(p)
    rep.sign_mismatch = int(smis.sum())
    rep.sign_bad = int((smis & (pa >= SIGN_WINDOW)).sum())
    rep.sign_bad_normalized = int((smis & (pa / np.sqrt(d) >= SIGN_WINDOW)).sum())
    rep.decision_keys = int((cmis.any(axis=1) | smis.any(axis=1)).sum())
    rep.idx, rep.beta = slots, lib_beta
    rep.nonfinite = int((~np.isfinite(norms)).sum() + (~np.isfinite(rnorms)).sum())
    rep.norm_bad = int((~_within(np.abs(norms - pq.norms), d * 2.0 ** -24 * pq.norms)).sum())
    rep.rnorm_bad = int((~_within(np.abs(rnorms - rn), np.sqrt(d) * 1e-6 + d * 2.0 ** -24 * rn)).sum())
    if rep.code_bad:
        i = np.argwhere(cmis & (dist >= CODE_WINDOW))[0]
        rep.worst["code"] = (tuple(int(x) for x in i), float(dist[tuple(i)]))
    if rep.sign_bad:
        i = np.argwhere(smis & (pa >= SIGN_WINDOW))[0]
        rep.worst["sign"] = (tuple(int(x) for x in i), float(pa[tuple(i)]))
    return rep


def e2e_scores_polar(pp, rep, queries, norms, rows=slice(None)):
    """End-to-end score reference for polar keys ``rows``: the oracle's
    estimator on the library's codes and signs, the oracle's norms and the
    reference rho."""
    from . import polar
    codes = [c[rows] for c in rep.reference["codes"]]
    return polar.scores(pp, queries, codes, rep.beta[rows], norms, rep.reference["rnorms"][rows])


def _ratio(err, tol):
    """err / tol with NaN and infinities mapped to inf."""
    r = np.asarray(err, dtype=np.float64) / np.maximum(tol, 1e-300)
    return np.where(np.isfinite(r), r, np.inf)


def score_violations(s_gpu, s_ref, queries, norms, keep=None):
    """(count of scores outside 1e-3 ||q|| n_k, worst error / tolerance);
    s arrays are (m, n).  A non-finite score counts as outside."""
    s_gpu = np.asarray(s_gpu, dtype=np.float64)
    s_ref = np.asarray(s_ref, dtype=np.float64)
    qn = np.linalg.norm(np.asarray(queries, dtype=np.float64), axis=1)
    tol = SCORE_TOL * qn[:, None] * np.asarray(norms, dtype=np.float64)[None, :]
    err = np.abs(s_gpu - s_ref)
    bad = ~_within(err, tol)
    ratio = _ratio(err, tol)
    if keep is not None:
        keep = np.asarray(keep)
        bad = bad[:, keep]
        ratio = ratio[:, keep]
    return int(bad.sum()), float(ratio.max()) if ratio.size else 0.0


def dequant_violations(k_gpu, k_ref):
    """(count of keys outside ||k_gpu - k|| <= 1e-5 ||k||, worst ratio); a
    non-finite reconstruction counts as outside."""
    k_gpu = np.asarray(k_gpu, dtype=np.float64)
    k_ref = np.asarray(k_ref, dtype=np.float64)
    err = np.linalg.norm(k_gpu - k_ref, axis=1)
    err = np.where(np.isfinite(k_gpu).all(axis=1), err, np.inf)
    tol = DEQUANT_TOL * np.linalg.norm(k_ref, axis=1)
    bad = ~_within(err, tol)
    ratio = _ratio(err, tol)
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
        if not np.all(_within(np.abs(vals - s_ref[i, ids]), tol[ids])):
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
