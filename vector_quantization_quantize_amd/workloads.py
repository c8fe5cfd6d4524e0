"""Seeded synthetic inputs for the five reference workloads.

Input generation only: nothing here touches the method's arithmetic, so the
CPU oracle and the HIP path can both be fed from it.  Every array comes from
``numpy.random.Generator(PCG64(seed))`` in a fixed draw order; ``n`` may be
lowered for a smaller instance with the same distribution.

Workloads (all synthetic; no dataset is read):

* ``toy``          d=128, 3 bits; 4096 fp32 keys iid N(0,1) scaled per key by
                   lognormal(0, 0.5); 16 fp32 queries iid N(0,1).
* ``llama_decode`` d=128, 4 bits; batch 1, 8 KV heads x 32768 tokens of bf16
                   keys N(0,1) with 4 seeded outlier channels per head scaled
                   x10; 32 fp32 query heads, 4 per KV head, one token.
* ``long_context`` d=128, 3 bits; batch 4, 8 KV heads x 131072 tokens of bf16
                   keys from the llama_decode generator; 32 query heads per
                   batch entry.
* ``search_b2`` / ``search_b4``  d=200, 2 / 4 bits; 1e6 vectors N(0, diag(i^-1))
                   L2-normalised, 1e4 queries from the same law.  Stand-in for
                   a GloVe-200 nearest-neighbour benchmark.
* ``cone``         d=1536, 4 bits; 1e6 unit vectors
                   normalize(0.87 mu + 0.49 (B z / 8 + eps)) with mu a seeded
                   unit vector, B a seeded orthonormal 1536 x 64 basis,
                   z ~ N(0, I_64), eps ~ N(0, 0.01^2 I); 4096 queries the same.
"""
from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    d: int
    bits: int
    groups: int          # independent key sets (batch x KV heads)
    n: int               # keys per group
    nq: int              # queries per group
    key_dtype: str       # "f32" or "bf16"
    description: str

    @property
    def total_keys(self):
        return self.groups * self.n

    def scaled(self, n=None, nq=None, groups=None):
        return replace(self, n=n or self.n, nq=nq or self.nq, groups=groups or self.groups)


WORKLOADS = {
    "toy": Workload("toy", 128, 3, 1, 4096, 16, "f32",
                    "d=128, 3 bits, 4096 fp32 keys N(0,1) x lognormal(0,0.5), 16 queries"),
    "llama_decode": Workload("llama_decode", 128, 4, 8, 32768, 4, "bf16",
                             "d=128, 4 bits, 8 KV heads x 32768 bf16 keys (4 outlier channels x10), "
                             "32 query heads (GQA 4), one decode step"),
    "long_context": Workload("long_context", 128, 3, 32, 131072, 4, "bf16",
                             "d=128, 3 bits, batch 4 x 8 KV heads x 131072 bf16 keys, 32 query heads "
                             "per batch entry (GQA 4)"),
    "search_b2": Workload("search_b2", 200, 2, 1, 1000000, 10000, "f32",
                          "d=200, 2 bits, 1e6 anisotropic unit vectors, 1e4 queries"),
    "search_b4": Workload("search_b4", 200, 4, 1, 1000000, 10000, "f32",
                          "d=200, 4 bits, 1e6 anisotropic unit vectors, 1e4 queries"),
    "cone": Workload("cone", 1536, 4, 1, 1000000, 4096, "f32",
                     "d=1536, 4 bits, 1e6 unit vectors in a narrow cone, 4096 queries"),
}


def _rng(seed, stream):
    return np.random.Generator(np.random.PCG64([int(seed), int(stream)]))


def _to_bf16_values(x):
    """Round float32 to bfloat16 (round to nearest even); return float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).copy()
    # finite inputs only: u + 0x8000 cannot wrap below the NaN range
    u += ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    u &= np.uint32(0xFFFF0000)
    return u.view(np.float32)


def _unit_rows(x):
    return x / np.linalg.norm(x, axis=1, keepdims=True)


def keys(w: Workload, seed=0, start=0, count=None):
    """Keys [groups * n, d] as float32 values (bf16-exact for bf16 workloads).

    ``start`` / ``count`` select a contiguous slice of the flattened
    [groups][n] key list without generating the rest (chunked draws)."""
    total = w.total_keys
    count = total - start if count is None else count
    assert 0 <= start and start + count <= total
    if w.name == "toy":
        rs = _rng(seed, 1)
        k = rs.standard_normal((w.total_keys, w.d)).astype(np.float32)
        scale = np.exp(0.5 * rs.standard_normal((w.total_keys, 1))).astype(np.float32)
        return (k * scale)[start:start + count]
    if w.name in ("llama_decode", "long_context"):
        return _gqa_keys(w, seed, start, count)
    if w.name.startswith("search"):
        return _chunked(w, seed, start, count, _search_chunk)
    if w.name == "cone":
        return _chunked(w, seed, start, count, _cone_chunk)
    raise KeyError(w.name)


_CHUNK = 65536


def _chunked(w, seed, start, count, fn):
    out = np.empty((count, w.d), dtype=np.float32)
    first = start // _CHUNK
    last = (start + count - 1) // _CHUNK if count else first - 1
    pos = 0
    for c in range(first, last + 1):
        block = fn(w, seed, c)
        lo = max(start - c * _CHUNK, 0)
        hi = min(start + count - c * _CHUNK, _CHUNK)
        out[pos:pos + hi - lo] = block[lo:hi]
        pos += hi - lo
    return out


def _search_chunk(w, seed, c):
    rs = _rng(seed, 1000 + c)
    scale = np.arange(1, w.d + 1, dtype=np.float64) ** -0.5
    x = rs.standard_normal((_CHUNK, w.d)) * scale[None, :]
    return _unit_rows(x).astype(np.float32)


def _cone_frame(w, seed):
    rs = _rng(seed, 7)
    mu = rs.standard_normal(w.d)
    mu /= np.linalg.norm(mu)
    basis, _ = np.linalg.qr(rs.standard_normal((w.d, 64)))
    return mu, basis


def _cone_rows(w, rs, count, mu, basis):
    z = rs.standard_normal((count, 64))
    eps = 0.01 * rs.standard_normal((count, w.d))
    g = z @ basis.T / 8.0 + eps
    return _unit_rows(0.87 * mu[None, :] + 0.49 * g).astype(np.float32)


def _cone_chunk(w, seed, c):
    mu, basis = _cone_frame(w, seed)
    return _cone_rows(w, _rng(seed, 2000 + c), _CHUNK, mu, basis)


def _gqa_keys(w, seed, start, count):
    """bf16 keys N(0,1), 4 distinct seeded outlier channels per KV head x10.

    Keys of group g (= batch * 8 + head) come from their own generator stream
    in chunks of 65536 tokens, so any slice is generated independently (and
    chunks are drawn on a thread pool)."""
    heads = 8
    out = np.empty((count, w.d), dtype=np.float32)
    tasks = []
    pos = 0
    key = start
    while pos < count:
        g = key // w.n
        t = key - g * w.n
        c = t // _CHUNK
        lo = t - c * _CHUNK
        take = min(_CHUNK - lo, w.n - t, count - pos)
        tasks.append((g, c, lo, take, pos))
        pos += take
        key += take

    def run(task):
        g, c, lo, take, at = task
        ch = _rng(seed, 50 + g % heads).choice(w.d, size=4, replace=False)
        rs = _rng(seed, 100000 + g * 4096 + c)
        block = rs.standard_normal((min(_CHUNK, w.n - c * _CHUNK), w.d), dtype=np.float32)
        block[:, ch] *= 10.0
        out[at:at + take] = _to_bf16_values(block[lo:lo + take])

    if len(tasks) == 1:
        run(tasks[0])
    else:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=8) as ex:
            list(ex.map(run, tasks))
    return out


def queries(w: Workload, seed=0):
    """Queries [groups, nq, d] float32."""
    if w.name == "cone":
        mu, basis = _cone_frame(w, seed)
        q = _cone_rows(w, _rng(seed, 3), w.groups * w.nq, mu, basis)
        return q.reshape(w.groups, w.nq, w.d)
    rs = _rng(seed, 2)
    if w.name.startswith("search"):
        scale = np.arange(1, w.d + 1, dtype=np.float64) ** -0.5
        q = _unit_rows(rs.standard_normal((w.groups * w.nq, w.d)) * scale[None, :])
        return q.astype(np.float32).reshape(w.groups, w.nq, w.d)
    return rs.standard_normal((w.groups, w.nq, w.d)).astype(np.float32)
