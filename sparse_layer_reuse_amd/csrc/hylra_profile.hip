// Offline profiling kernel of HyLRA for gfx950: the similarity matrix of the
// per-layer top-k index sets.
//
// Method: "HyLRA: Hybrid Layer Reuse Attention for Efficient Long-Context
// Inference", technical summary 2.2: the policy program runs on a
// lower-triangular matrix M built offline from the overlap ratio of the top-k
// indices of layer pairs.  Here a slice is (profiling step, sequence, KV
// head); for source layer i <= target layer j its ratio is
// |I_i n I_j| / |I_j| (-1 entries are padding, a slice with an empty target
// set is skipped), and M[j][i] is the mean of the ratio over slices.
//
// One workgroup per target layer j, 4 wavefronts.  Per slice (in order) the
// sets of layers 0..j are staged in LDS; wavefront w takes the sources
// i = w, w+4, ...: its lanes hold the target's ids 64 at a time, each looks
// its id up in I_i by binary search (sets are ascending), and a ballot counts
// the hits.  Ratios are summed in float64 in slice order, so the result does
// not depend on scheduling.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hylra_internal.h"

namespace hylra {
namespace {

constexpr int kProfileThreads = 256;
constexpr int kProfileWaves = kProfileThreads / 64;

// Number of leading ids >= 0 of an ascending, -1 padded set of k entries
// (wavefront-uniform; every lane computes it).
__device__ __forceinline__ int valid_count(const int32_t *set, int k) {
  int n = 0;
  for (int t0 = 0; t0 < k; t0 += 64) {
    const int t = t0 + (int)(threadIdx.x & 63);
    n += __builtin_popcountll(__ballot(t < k && set[t] >= 0));
  }
  return n;
}

// Whether x occurs in set[0..n) (ascending).
__device__ __forceinline__ bool contains(const int32_t *set, int n, int32_t x) {
  int lo = 0, hi = n;  // first position with set[pos] >= x lies in [lo, hi]
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (set[mid] < x)
      lo = mid + 1;
    else
      hi = mid;
  }
  return lo < n && set[lo] == x;
}

__global__ __launch_bounds__(kProfileThreads) void overlap_rows(OverlapArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  double *sums = reinterpret_cast<double *>(smem);                     // [L]
  int32_t *sets = reinterpret_cast<int32_t *>(smem + 8 * a.layers);   // [j + 1][k]
  const int j = blockIdx.x;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int i = threadIdx.x; i <= j; i += kProfileThreads) sums[i] = 0.0;
  int used = 0;
  for (int p = 0; p < a.steps; ++p) {
    for (int s = 0; s < a.slices; ++s) {
      __syncthreads();  // the previous slice's sets are no longer read
      for (int e = threadIdx.x; e < (j + 1) * a.k; e += kProfileThreads) {
        const int l = e / a.k, t = e - l * a.k;
        sets[e] = a.idx[(((int64_t)p * a.layers + l) * a.slices + s) * a.k + t];
      }
      __syncthreads();
      const int32_t *tgt = sets + (int64_t)j * a.k;
      const int nt = valid_count(tgt, a.k);
      if (nt == 0) continue;  // uniform across the workgroup
      ++used;
      for (int i = w; i <= j; i += kProfileWaves) {
        const int32_t *src = sets + (int64_t)i * a.k;
        const int ns = valid_count(src, a.k);
        int hits = 0;
        for (int t0 = 0; t0 < nt; t0 += 64) {
          const int t = t0 + lane;
          const bool hit = t < nt && contains(src, ns, tgt[t]);
          hits += __builtin_popcountll(__ballot(hit));
        }
        if (lane == 0) sums[i] += (double)hits / (double)nt;
      }
    }
  }
  __syncthreads();
  float *row = a.M + (int64_t)j * a.layers;
  for (int i = threadIdx.x; i < a.layers; i += kProfileThreads)
    row[i] = (i <= j && used > 0) ? (float)(sums[i] / (double)used) : 0.f;
}

}  // namespace

size_t overlap_smem_bytes(int layers, int k) {
  return (size_t)8 * layers + (size_t)4 * layers * k;
}

int launch_overlap(const OverlapArgs &a, void *stream) {
  hipLaunchKernelGGL(overlap_rows, dim3(a.layers), dim3(kProfileThreads),
                     overlap_smem_bytes(a.layers, a.k), static_cast<hipStream_t>(stream), a);
  return (int)hipGetLastError();
}

}  // namespace hylra
