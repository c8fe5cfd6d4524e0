"""CPU oracle for the TurboQuant quantize / score path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this
package: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` use it.  It shares no code, tables or constants generator with
the HIP library; both are written independently from the same description.

Everything is plain numpy / scipy in float64, one step per stage of the
method, in the order the pages give:

* ``rng``       - counter-based SplitMix64 + Box-Muller normal draws (the
                  method's random matrices are derived from a seed).
* ``params``    - Haar rotation Pi, Gaussian projection G, Lloyd-Max codebook
                  for the coordinate marginal of a rotated unit vector.
* ``tq``        - quantize (normalize, rotate, bucketize, residual, QJL
                  signs), bit-plane packing, the asymmetric score and the
                  stage-1 reconstruction.

Sources are cited by page title and section:

* "TurboQuant digest" (juejin.cn), section 2: random rotation, then scalar
  quantization carrying most of the bit budget, then about one bit of QJL
  sign sketch on the residual with an asymmetric estimator.
* "TurboQuant tutorial" (gitcode.csdn.net), sections PolarQuant and QJL:
  the 4-D rotation example, nearest allowed value, residual, Gaussian
  projection, sign bits (positive -> 1), the unbiased correction, and the
  2+1 / 3+1 bit split.
* "TurboQuant deep review" (freelamp.com), sections on the breakthrough and
  on error compensation: random orthogonal preconditioning; zero-bias
  estimate from 1-bit residual signs against a high-precision query.
"""
