"""Quantize, pack, score and reconstruct (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Each function follows one stage of the method in the pages' order.  All
arithmetic is float64; the two decisions that produce integers (the stage-1
code and the QJL sign) are taken on the float32 rounding of the float64
value, the precision in which the library takes them.

Stages (page, section):

1. norm and direction: the length of the vector is kept at higher precision
   and only its direction is quantized ("TurboQuant tutorial", Cartesian to
   polar part of the PolarQuant section).  n = ||k||, u = k / n (u = 0 when
   n = 0, so the pipeline runs literally on a zero key).
2. rotation: z = Pi u ("TurboQuant digest" section 2; "TurboQuant tutorial",
   PolarQuant 4-D example).
3. scalar quantization: each z_j becomes the nearest allowed value; the
   index is the number of thresholds t_i <= z_j (a tie goes to the upper
   cell) ("TurboQuant tutorial", QJL section, first paragraph).
4. residual: r = z - c[idx], rho = ||r|| ("TurboQuant tutorial", QJL step 1).
5. Gaussian projection and 1-bit signs: p = G r, beta_j = 1 iff p_j > 0
   ("TurboQuant tutorial", QJL steps 1-2: positive -> 1, negative -> 0;
   p_j = 0 gives 0).
6. asymmetric score of a full-precision query q against the stored key:
   v = Pi q, w = G v (= S q with S = G Pi), and
       s = n * ( <v, c[idx]> + rho * sqrt(pi/2) / d * <w, 2 beta - 1> )
   ("TurboQuant digest" section 2 and "TurboQuant deep review", error
   compensation section: 1-bit residual signs combined with a high-precision
   query give an estimate with zero bias; the constant sqrt(pi/2)/d is what
   makes it unbiased: E[x sign(y)] = sqrt(2/pi) Cov(x, y) / sd(y)).
7. stage-1 reconstruction: k_hat = n * Pi^T c[idx] ("TurboQuant tutorial",
   end of the polar part: codes plus the kept length map back to a vector).
8. search: brute-force scores of every query against every stored key, then
   the k best keys per query ("TurboQuant digest" section 3, the vector
   search comparison by recall).  Best = largest estimated score; equal
   scores go in ascending key order (the pages do not order ties).  Recall
   compares those keys with the k best by the exact inner product of the
   unquantized vectors: recall@k is the shared fraction, and Recall@1@k the
   share of queries whose exact best key is among the k found.

9. reconstruction with the correction: the score is linear in q
   (<w, 2 beta - 1> = <G Pi q, 2 beta - 1> = <q, Pi^T G^T (2 beta - 1)>), so
   one vector per key reproduces it for every query,
       k_tilde = n * Pi^T ( c[idx] + rho * sqrt(pi/2) / d * G^T (2 beta - 1) )
   ("TurboQuant deep review", error compensation section: the corrected
   estimate is unbiased, and this is the vector it is the inner product
   with).
10. decode attention over a compressed cache: the cache holds key-value
   pairs ("Why KV-cache compression works", section 2: the method quantizes
   the KV cache; "TurboQuant tutorial", glossary: q asks, k identifies, v
   carries the content).  Keys are scored with the stage-6 estimate;
   values are stored with stage 1 only and read back by the stage-7
   reconstruction (the QJL bit serves inner products with a query, which
   a value never takes part in).  For each query
       o = sum_t softmax_t(scale * s_t) * v_hat_t,
   with the caller's scale (1/sqrt(d) in the usual attention) and every
   stored token visible; also lse = log sum_t exp(scale * s_t).  With no
   tokens o = 0 and lse = -inf.

11. fractional widths (2.5 or 3.5 bits per coordinate): the rotated
   coordinates are split in two groups, the first hi with one more index
   bit (a Lloyd-Max set with twice the levels for the same coordinate law)
   and the rest with bits - 1; stages 3, 4, 6, 7 and 9 take each
   coordinate's level from its own set.  The pages quote these operating
   points ("TurboQuant digest", section 4: 3.5 bits per channel with no
   loss of quality, 2.5 bits with a marginal one) without the mechanism;
   this split of the rotated coordinates into two widths is the reading
   taken.

Packed layout (bit planes): ``codes[n][B][W]`` and ``signs[n][W]`` as
uint32 with W = ceil(d / 32); bit p of the index of coordinate j is bit
(j mod 32) of word (j div 32) of plane p (LSB first); padding bits are 0.
Stored values use token blocks instead: ``vcodes[ceil(n/32)][B][32 W]``
(uint32 words, read here as little-endian bytes: 128 B W bytes per block
of 32 tokens; tokens past n and coordinates past d give index 0).
Coordinates come in groups of 128 (4 words of the key layout; the last
group holds G = W mod 4 words when that is not 0); group g's 512 B G bytes
start at byte 512 B g of the block.  For coordinate 128 g + r (r < 32 G)
and token octet o (tokens 32 b + 8 o .. + 7), the B-byte little-endian
integer X at byte ((r mod 16) + 16 o) * 2 G B + (r div 16) * B of the
group holds, for token 8 o + t and plane p, bit p of the token's index at
bit (t div E) * B E + p E + (t mod E), with E = 8, 4, 2, 2 for B = 1, 2,
3, 4: each run of B E bits is the index bits of E consecutive tokens.
"""
from dataclasses import dataclass

import numpy as np

from .params import Params

QJL_CONST = np.sqrt(np.pi / 2.0)


@dataclass
class Quantized:
    """Unpacked quantizer output for n keys plus the pre-decision values."""
    idx: np.ndarray      # (n, d) int64 codebook indices
    beta: np.ndarray     # (n, d) bool QJL sign bits
    norms: np.ndarray    # (n,) float64, ||k||
    rnorms: np.ndarray   # (n,) float64, ||r||
    z: np.ndarray        # (n, d) float64 rotated unit-vector coordinates
    p: np.ndarray        # (n, d) float64 projected residual


def normalize(keys):
    """Stage 1: (norms, unit directions); zero keys give a zero direction."""
    k = np.asarray(keys, dtype=np.float64)
    norms = np.sqrt(np.sum(k * k, axis=1))
    safe = np.where(norms > 0.0, norms, 1.0)
    u = np.where((norms > 0.0)[:, None], k / safe[:, None], 0.0)
    return norms, u


def rotate(params: Params, u):
    """Stage 2: z = Pi u for each row u."""
    return u @ params.pi.T


def bucketize(params: Params, z):
    """Stage 3: index = #{i : t_i <= fp32(z)} (upper cell on a tie), with
    the finer thresholds for coordinates below ``params.hi``."""
    z32 = np.asarray(z, dtype=np.float64).astype(np.float32).astype(np.float64)
    h = params.hi
    if h == 0:
        return np.searchsorted(params.thresholds, z32, side="right").astype(np.int64)
    fine = np.searchsorted(params.thresholds_hi, z32[:, :h], side="right")
    base = np.searchsorted(params.thresholds, z32[:, h:], side="right")
    return np.concatenate([fine, base], axis=1).astype(np.int64)


def levels_of(params: Params, idx):
    """c[idx] for an (n, d) index array, each coordinate from its own level
    set (the finer one below ``params.hi``)."""
    idx = np.asarray(idx)
    h = params.hi
    if h == 0:
        return params.centroids[idx]
    return np.concatenate([params.centroids_hi[idx[:, :h]], params.centroids[idx[:, h:]]], axis=1)


def residual(params: Params, z, idx):
    """Stage 4: r = z - c[idx] and its norm."""
    r = z - levels_of(params, idx)
    return r, np.sqrt(np.sum(r * r, axis=1))


def project_signs(params: Params, r):
    """Stage 5: p = G r and beta = [fp32(p) > 0]."""
    p = r @ params.g.T
    beta = p.astype(np.float32) > 0
    return p, beta


def quantize(params: Params, keys):
    """Stages 1-5 for a batch of keys of shape (n, d)."""
    keys = np.asarray(keys, dtype=np.float64)
    assert keys.ndim == 2 and keys.shape[1] == params.d
    norms, u = normalize(keys)
    z = rotate(params, u)
    idx = bucketize(params, z)
    r, rnorms = residual(params, z, idx)
    p, beta = project_signs(params, r)
    return Quantized(idx, beta, norms, rnorms, z, p)


def query_transform(params: Params, queries):
    """Stage 6, query side: v = Pi q and w = G v for each row q."""
    q = np.asarray(queries, dtype=np.float64)
    v = q @ params.pi.T
    w = v @ params.g.T
    return v, w


def scores(params: Params, queries, idx, beta, norms, rnorms):
    """Stage 6: (m, n) matrix of estimates <q_a, k_hat_b>."""
    v, w = query_transform(params, queries)
    chat = levels_of(params, idx)                             # (n, d)
    signs = np.where(np.asarray(beta), 1.0, -1.0)             # (n, d)
    stage1 = v @ chat.T                                       # (m, n)
    qjl = w @ signs.T                                         # (m, n)
    scale = np.asarray(rnorms, dtype=np.float64) * QJL_CONST / params.d
    return np.asarray(norms, dtype=np.float64)[None, :] * (stage1 + scale[None, :] * qjl)


def dequant_mse(params: Params, idx, norms):
    """Stage 7: k_hat = n * Pi^T c[idx] for each key."""
    chat = levels_of(params, idx)
    return np.asarray(norms, dtype=np.float64)[:, None] * (chat @ params.pi)


def dequant_prod(params: Params, idx, beta, norms, rnorms):
    """Stage 9: k_tilde = n Pi^T (c[idx] + rho sqrt(pi/2)/d G^T (2 beta - 1))
    for each key (rows of the result)."""
    chat = levels_of(params, idx)                             # (n, d)
    signs = np.where(np.asarray(beta), 1.0, -1.0)             # (n, d)
    scale = np.asarray(rnorms, dtype=np.float64) * QJL_CONST / params.d
    corr = scale[:, None] * (signs @ params.g)                # row b: (G^T s_b)^T
    return np.asarray(norms, dtype=np.float64)[:, None] * ((chat + corr) @ params.pi)


def attention(key_params: Params, value_params: Params, queries, k_idx, k_beta, k_norms, k_rnorms, v_idx,
              v_norms, scale):
    """Stage 10: (o (m, d), lse (m,)) of m queries over n stored tokens."""
    q = np.asarray(queries, dtype=np.float64)
    m, n = q.shape[0], np.asarray(v_norms).shape[0]
    if n == 0:
        return np.zeros((m, value_params.d)), np.full(m, -np.inf)
    s = float(scale) * scores(key_params, q, k_idx, k_beta, k_norms, k_rnorms)   # (m, n)
    top = s.max(axis=1, keepdims=True)
    e = np.exp(s - top)
    total = e.sum(axis=1)
    probs = e / total[:, None]
    vhat = dequant_mse(value_params, v_idx, v_norms)          # (n, d)
    return probs @ vhat, top[:, 0] + np.log(total)


def topk(scores, k):
    """Stage 8: (indices, scores) of the k largest entries of each row of an
    (m, n) score matrix, best first; equal scores in ascending column order.
    k is capped at n."""
    s = np.asarray(scores, dtype=np.float64)
    k = min(int(k), s.shape[1])
    order = np.argsort(-s, axis=1, kind="stable")[:, :k]
    return order, np.take_along_axis(s, order, axis=1)


def exact_inner_products(queries, keys):
    """<q, k> of the unquantized vectors, float64, (m, n)."""
    return np.asarray(queries, dtype=np.float64) @ np.asarray(keys, dtype=np.float64).T


def recall_at_k(found, exact):
    """Mean over rows of |found_row & exact_row| / k (both (m, k) index arrays)."""
    found = np.asarray(found)
    exact = np.asarray(exact)
    k = exact.shape[1]
    return float(np.mean([len(set(f.tolist()) & set(e.tolist())) / k for f, e in zip(found, exact)]))


def recall_1_at_k(found, exact_best):
    """Share of rows whose exact best key (exact_best, shape (m,)) is in the
    row's found indices."""
    found = np.asarray(found)
    return float(np.mean([b in set(f.tolist()) for f, b in zip(found, np.asarray(exact_best))]))


# ----------------------------------------------------------------------------
# bit-plane packing
# ----------------------------------------------------------------------------

def words_per_plane(d):
    return (d + 31) // 32


def pack_bits(bits):
    """(n, d) bool -> (n, W) uint32, coordinate j at word j//32, bit j%32."""
    bits = np.asarray(bits, dtype=bool)
    n, d = bits.shape
    w = words_per_plane(d)
    padded = np.zeros((n, w * 32), dtype=np.uint64)
    padded[:, :d] = bits
    weights = np.uint64(1) << np.arange(32, dtype=np.uint64)
    words = (padded.reshape(n, w, 32) * weights[None, None, :]).sum(axis=2)
    return words.astype(np.uint32)


def unpack_bits(words, d):
    """(n, W) uint32 -> (n, d) bool (inverse of pack_bits)."""
    words = np.asarray(words, dtype=np.uint32)
    n, w = words.shape
    shifts = np.arange(32, dtype=np.uint32)
    bits = (words[:, :, None] >> shifts[None, None, :]) & np.uint32(1)
    return bits.reshape(n, w * 32)[:, :d].astype(bool)


def pack_codes(idx, code_bits):
    """(n, d) indices -> (n, B, W) uint32 bit planes (plane p = bit p)."""
    idx = np.asarray(idx, dtype=np.int64)
    planes = [pack_bits((idx >> p) & 1) for p in range(code_bits)]
    return np.stack(planes, axis=1)


def unpack_codes(codes, d):
    """(n, B, W) uint32 -> (n, d) indices."""
    codes = np.asarray(codes, dtype=np.uint32)
    n, b, _ = codes.shape
    idx = np.zeros((n, d), dtype=np.int64)
    for p in range(b):
        idx |= unpack_bits(codes[:, p, :], d).astype(np.int64) << p
    return idx


def pack_codes_split(idx, code_bits, hi):
    """Fractional widths: (n, d) indices (coordinates below hi may use one
    more bit) -> (n, B W + ceil(hi / 32)) uint32: planes 0 .. B-1 over all
    coordinates as in pack_codes, one after another, then plane B over the
    coordinates 0 .. hi-1 only."""
    idx = np.asarray(idx, dtype=np.int64)
    n = idx.shape[0]
    base = pack_codes(idx & ((1 << code_bits) - 1), code_bits).reshape(n, -1)
    if hi == 0:
        return base
    top = pack_bits(((idx[:, :hi] >> code_bits) & 1).astype(bool))
    return np.concatenate([base, top], axis=1)


def unpack_codes_split(codes, d, code_bits, hi):
    """Inverse of pack_codes_split."""
    codes = np.asarray(codes, dtype=np.uint32)
    n = codes.shape[0]
    w = words_per_plane(d)
    idx = unpack_codes(codes[:, :code_bits * w].reshape(n, code_bits, w), d)
    if hi:
        idx[:, :hi] |= unpack_bits(codes[:, code_bits * w:], hi).astype(np.int64) << code_bits
    return idx


def pack(params: Params, qz: Quantized):
    """Packed buffers (codes, signs, norms fp32, rnorms fp32) of a batch;
    codes as pack_codes_split when the parameters have fractional widths."""
    codes = (pack_codes_split(qz.idx, params.code_bits, params.hi) if params.hi
             else pack_codes(qz.idx, params.code_bits))
    return (codes, pack_bits(qz.beta), qz.norms.astype(np.float32), qz.rnorms.astype(np.float32))


def value_group_of_e(code_bits):
    """Tokens per index run in the value layout: 8, 4, 2, 2 for B = 1..4."""
    return {1: 8, 2: 4, 3: 2, 4: 2}[code_bits]


def value_slot(d, code_bits):
    """(32 W, 4) int: byte offset, within a block, of the B-byte integer X
    for coordinate j and token octet o (see the module docstring)."""
    w = words_per_plane(d)
    pos = np.empty((32 * w, 4), dtype=np.int64)
    for j in range(32 * w):
        g, r = divmod(j, 128)
        gw = min(4, w - 4 * g)                      # words in this group
        for o in range(4):
            pos[j, o] = 512 * code_bits * g + ((r % 16) + 16 * o) * 2 * gw * code_bits + (r // 16) * code_bits
    return pos


def pack_values(idx, code_bits):
    """(n, d) value indices -> (ceil(n/32), B, 32 W) uint32 token blocks in
    the value layout (module docstring)."""
    idx = np.asarray(idx, dtype=np.int64)
    n, d = idx.shape
    nb = (n + 31) // 32
    dp = 32 * words_per_plane(d)
    e = value_group_of_e(code_bits)
    slot = value_slot(d, code_bits)
    padded = np.zeros((nb * 32, dp), dtype=np.int64)
    padded[:n, :d] = idx
    out = np.zeros((nb, 4 * code_bits * dp), dtype=np.uint8)
    for b in range(nb):
        for o in range(4):
            toks = padded[32 * b + 8 * o:32 * b + 8 * o + 8]          # (8 tokens, dp)
            x = np.zeros(dp, dtype=np.uint64)
            for t in range(8):
                for p in range(code_bits):
                    bit = (toks[t] >> p) & 1
                    x |= bit.astype(np.uint64) << np.uint64((t // e) * code_bits * e + p * e + t % e)
            for k in range(code_bits):
                out[b, slot[:, o] + k] = (x >> np.uint64(8 * k)) & np.uint64(0xFF)
    return out.view("<u4").reshape(nb, code_bits, dp)


def unpack_values(vcodes, n, d):
    """Inverse of pack_values: (n, d) indices."""
    vcodes = np.ascontiguousarray(np.asarray(vcodes, dtype=np.uint32))
    nb, code_bits, dp = vcodes.shape
    raw = vcodes.reshape(nb, code_bits * dp).view("<u1").astype(np.uint64)
    e = value_group_of_e(code_bits)
    slot = value_slot(d, code_bits)
    idx = np.zeros((nb * 32, dp), dtype=np.int64)
    for b in range(nb):
        for o in range(4):
            x = np.zeros(dp, dtype=np.uint64)
            for k in range(code_bits):
                x |= raw[b, slot[:, o] + k] << np.uint64(8 * k)
            for t in range(8):
                for p in range(code_bits):
                    bit = (x >> np.uint64((t // e) * code_bits * e + p * e + t % e)) & np.uint64(1)
                    idx[32 * b + 8 * o + t] |= bit.astype(np.int64) << p
    return idx[:n, :d]
