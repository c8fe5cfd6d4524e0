// Running top-k of the search entry point ("TurboQuant digest", section 3:
// brute-force scores, compared by recall): merges one chunk of scores per
// query into that query's list of the k best keys so far.  The chunk holds
// either consecutive keys (scores only) or (score, key) pairs, such as the
// per-block lists of the matrix-core search kernel.
//
// One wave per query.  Lane j holds entry j of the list (best first: larger
// score, then smaller key index).  The wave reads the chunk 64 scores at a
// time; a lane's score is a candidate when it beats the list's k-th entry
// (any score while the list is not full).  Candidates are rare once the list
// has filled, so they are inserted one at a time: the insert position is the
// number of entries that beat the candidate (one ballot), and the entries
// from there on move down one lane.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "tq_internal.h"

namespace tqdev {
namespace {

constexpr int kWavesPerBlock = 4;
constexpr int64_t kNoIndex = INT64_MAX;

// (sa, ia) ranks before (sb, ib)
__device__ __forceinline__ bool better(float sa, int64_t ia, float sb, int64_t ib) {
  return sa > sb || (sa == sb && ia < ib);
}

__device__ __forceinline__ float read_lane(float x, int j) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), j));
}

__device__ __forceinline__ int64_t read_lane(int64_t x, int j) {
  const uint64_t u = static_cast<uint64_t>(x);
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(u & 0xFFFFFFFFu), j);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(u >> 32), j);
  return static_cast<int64_t>((uint64_t(hi) << 32) | lo);
}

// value of lane - 1 (lane 0 keeps its own)
__device__ __forceinline__ float from_prev(float x) { return __shfl_up(x, 1); }
__device__ __forceinline__ int64_t from_prev(int64_t x) {
  const uint64_t u = static_cast<uint64_t>(x);
  const uint32_t lo = __shfl_up(static_cast<unsigned>(u & 0xFFFFFFFFu), 1);
  const uint32_t hi = __shfl_up(static_cast<unsigned>(u >> 32), 1);
  return static_cast<int64_t>((uint64_t(hi) << 32) | lo);
}

__global__ void __launch_bounds__(64 * kWavesPerBlock)
topk_merge_kernel(const float* __restrict__ chunk, const int64_t* __restrict__ chunk_i, int64_t nq,
                  int64_t csize, int64_t c0, int k, float* __restrict__ list_s, int64_t* __restrict__ list_i,
                  int last,
                  float* __restrict__ out_s, int64_t* __restrict__ out_i) {
  const int lane = threadIdx.x & 63;
  const int64_t q = int64_t(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6);
  if (q >= nq) return;  // the whole wave
  // entries held: every key seen so far entered the list while it was not
  // full, so the count is min(k, keys before this chunk)
  int cnt = c0 < k ? static_cast<int>(c0) : k;
  float ls = -INFINITY;
  int64_t li = kNoIndex;
  if (lane < cnt) {
    ls = list_s[q * k + lane];
    li = list_i[q * k + lane];
  }
  float ts = -INFINITY;  // the k-th entry once the list is full
  int64_t ti = kNoIndex;
  if (cnt == k) {
    ts = read_lane(ls, k - 1);
    ti = read_lane(li, k - 1);
  }
  const float* row = chunk + q * csize;
  const int64_t* row_i = chunk_i ? chunk_i + q * csize : nullptr;
  for (int64_t b = 0; b < csize; b += 64) {
    const int64_t t = b + lane;
    const bool in = t < csize;
    const float s = in ? row[t] : -INFINITY;
    const int64_t idx = !in ? kNoIndex : row_i ? row_i[t] : c0 + t;
    uint64_t mask = __ballot(better(s, idx, ts, ti));
    while (mask) {
      const int j = __ffsll(static_cast<unsigned long long>(mask)) - 1;
      mask &= mask - 1;
      const float ns = read_lane(s, j);
      const int64_t ni = read_lane(idx, j);
      if (!better(ns, ni, ts, ti)) continue;  // the threshold rose meanwhile
      const int pos = __popcll(__ballot(lane < cnt && better(ls, li, ns, ni)));
      const float ps = from_prev(ls);
      const int64_t pi = from_prev(li);
      if (lane > pos) {
        ls = ps;
        li = pi;
      }
      if (lane == pos) {
        ls = ns;
        li = ni;
      }
      if (lane >= k) {  // an entry pushed past the k-th leaves the list
        ls = -INFINITY;
        li = kNoIndex;
      }
      cnt = cnt < k ? cnt + 1 : k;
      if (cnt == k) {
        ts = read_lane(ls, k - 1);
        ti = read_lane(li, k - 1);
      }
    }
  }
  if (lane < k) {
    if (last) {
      out_s[q * k + lane] = lane < cnt ? ls : -INFINITY;
      out_i[q * k + lane] = lane < cnt ? li : -1;
    } else {
      list_s[q * k + lane] = ls;
      list_i[q * k + lane] = li;
    }
  }
}

__global__ void fill_u32_kernel(unsigned int* __restrict__ p, int64_t n, unsigned int v) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

}  // namespace

hipError_t launch_fill_u32(unsigned int* p, int64_t n, unsigned int v, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(fill_u32_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream, p, n, v);
  return hipGetLastError();
}

hipError_t launch_topk_merge(const float* chunk, const int64_t* chunk_i, int64_t nq, int64_t csize, int64_t c0,
                             int k, float* list_s, int64_t* list_i, bool last, float* out_s, int64_t* out_i,
                             hipStream_t stream) {
  if (k < 1 || k > kTopkMax) return hipErrorInvalidValue;
  const int64_t blocks = (nq + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(topk_merge_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(64 * kWavesPerBlock), 0, stream,
                     chunk, chunk_i, nq, csize, c0, k, list_s, list_i, last ? 1 : 0, out_s, out_i);
  return hipGetLastError();
}

}  // namespace tqdev
