"""Counter-based normal draws for the method's seeded matrices (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages say only that the rotation is random and the projection Gaussian;
they fix no generator.  Both the oracle and the library implement the same
published generator independently, from this definition:

* SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014): with golden gamma ``g = 0x9E3779B97F4A7C15`` a
  generator whose state is ``s`` returns, on its i-th call (i = 1, 2, ...),
  ``fmix(s + i*g)`` where ``fmix`` is the 64-bit finalizer
  ``z ^= z>>30; z *= 0xBF58476D1CE4E5B9; z ^= z>>27; z *= 0x94D049BB133111EB;
  z ^= z>>31`` (all arithmetic mod 2**64).
* Stream ``k`` of seed ``seed`` is the SplitMix64 generator whose state is
  ``fmix(seed + (k+1)*g)``; counter ``c`` (0-based) of that stream is its
  (c+1)-th output.  Stream 0 feeds the rotation, stream 1 the projection.
* Normal pair ``i`` uses counters ``2i`` (a) and ``2i+1`` (b):
  ``u1 = ((a>>11)+1) * 2**-53`` in (0, 1], ``u2 = (b>>11) * 2**-53`` in
  [0, 1), ``R = sqrt(-2 ln u1)``; element ``2i`` is ``R cos(2 pi u2)`` and
  element ``2i+1`` is ``R sin(2 pi u2)`` (Box & Muller 1958).  An odd count
  drops the last sine.
* Random signs (stream 2, the randomized Hadamard rotation): sign ``j`` is
  -1 when bit 63 of counter ``j`` is set, else +1.
"""
import numpy as np

GAMMA = 0x9E3779B97F4A7C15
_MASK = (1 << 64) - 1


def fmix64(z):
    """SplitMix64 output finalizer on a uint64 array (wrapping arithmetic)."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
        z = z ^ (z >> np.uint64(31))
    return z


def splitmix64_sequence(state, count):
    """The first ``count`` outputs of a SplitMix64 generator with ``state``."""
    i = np.arange(1, count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        x = np.uint64(state & _MASK) + i * np.uint64(GAMMA)
    return fmix64(x)


def stream_state(seed, stream):
    """State of stream ``stream`` of ``seed`` (python ints, exact mod 2**64)."""
    x = (int(seed) + (int(stream) + 1) * GAMMA) & _MASK
    return int(fmix64(np.array([x], dtype=np.uint64))[0])


def uniform_bits(seed, stream, count):
    """Counters 0 .. count-1 of the stream as uint64."""
    return splitmix64_sequence(stream_state(seed, stream), count)


def normals(seed, stream, count):
    """``count`` standard normal draws (float64) of the given stream."""
    pairs = (count + 1) // 2
    bits = uniform_bits(seed, stream, 2 * pairs)
    a = bits[0::2]
    b = bits[1::2]
    u1 = ((a >> np.uint64(11)).astype(np.float64) + 1.0) * 2.0 ** -53
    u2 = (b >> np.uint64(11)).astype(np.float64) * 2.0 ** -53
    radius = np.sqrt(-2.0 * np.log(u1))
    theta = 2.0 * np.pi * u2
    out = np.empty(2 * pairs, dtype=np.float64)
    out[0::2] = radius * np.cos(theta)
    out[1::2] = radius * np.sin(theta)
    return out[:count]


def signs(seed, stream, count):
    """``count`` random signs (float64 +-1) of the given stream."""
    bits = uniform_bits(seed, stream, count)
    return np.where((bits >> np.uint64(63)) != 0, -1.0, 1.0)
