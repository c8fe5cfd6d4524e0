// Host-side parameter construction (float64, no HIP calls).
#pragma once
#include <cstddef>
#include <cstdint>

namespace tqhost {

// State of SplitMix64 stream `stream` of `seed`.
uint64_t stream_state(uint64_t seed, uint32_t stream);

// `count` standard normal draws of the stream, Box-Muller on counter pairs.
void normal_draws(uint64_t seed, uint32_t stream, size_t count, double* out);

// Householder QR of the row-major d x d matrix `a`; writes Q diag(sign(diag R))
// row-major into `q`.
void haar_from_gaussian(int d, const double* a, double* q);

// Lloyd-Max levels (ascending, symmetric) for the law of one coordinate of a
// uniform unit vector in R^d.  Returns 0 on convergence.
int lloyd_max_sphere(int d, int levels, double* c);

// Angle codebook of recursion level `level` (1 .. log2 d) of the polar
// stage: level 1 the uniform quantizer of [0, 2 pi), higher levels Lloyd-Max
// for the angle law of two 2^(level-1)-dimensional Gaussian blocks.
// levels: float[2^(bits-1)] ascending; thresholds: float[2^(bits-1) - 1]
// (float32 midpoints; level 1: the cell edges).  d a power of two.
// Returns 0, or < 0 on bad arguments / non-convergence.
int polar_level_codebook(int d, int bits, int level, float* levels, float* thresholds);

// Randomized Hadamard rotation H diag(sigma) / sqrt(d) (float[d*d] row-major):
// H[i][j] = (-1)^popcount(i & j) (Sylvester), sigma_j = -1 when bit 63 of
// counter j of stream 2 is set, else +1.  d a power of two in [2, 4096];
// returns 0, or -1 for another d.
int hadamard_rotation(int d, uint64_t seed, float* pi);

// Fill any of pi, g (float[d*d]), centroids (float[L]), thresholds
// (float[L-1]); NULL outputs are skipped.  g holds the stream-1 draws
// rounded to float16 precision.  Returns 0, or < 0 on bad
// arguments / non-convergence.
int build_params(int d, int bits, uint64_t seed, float* pi, float* g, float* centroids,
                 float* thresholds);

}  // namespace tqhost
