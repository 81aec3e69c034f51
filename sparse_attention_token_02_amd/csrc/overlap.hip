// Pairwise cross-layer overlap of top-k index sets for gfx950.
//
// What is computed (IndexCache deep-dive report, section 1.2: the overlap
// |T_i ∩ T_j| / k of the top-k sets of layers i and j): for N index tensors
// idx_i [L, k] (ascending, -1 padded) and the rows
// t = row_begin, row_begin + row_stride, ... < row_end,
//   C[i][j] = sum_t |T_i(t) ∩ T_j(t)|   (uint64).
// Integer counts summed with atomic adds: the result does not depend on the
// order in which rows are processed.
//
// A workgroup handles a strided subset of the rows.  The key range of a row,
// [0, largest index any layer holds in it] (at most [0, t] for a causal
// prefill row, [0, len_b) for a decode row), is cut into windows of 8192
// keys; for each window every layer's keys
// are set in an LDS bitmap (the range of each sorted list that falls in the
// window is found by binary search), then every thread ANDs and popcounts the
// bitmaps of its layer pairs and keeps the running counts in registers until
// the workgroup is done.
#include "device_common.hpp"
#include "kernels.hpp"

namespace dsa {

namespace {
constexpr int OV_NT = 256;
constexpr int OV_WBITS = 8192;
constexpr int OV_WWORDS = OV_WBITS / 32;
constexpr int OV_PPT = (OVERLAP_MAX_N * (OVERLAP_MAX_N + 1) / 2 + OV_NT - 1) / OV_NT;  // pairs per thread

__device__ __forceinline__ int lower_bound_i32(const int32_t* a, int n, int v) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] < v) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}
}  // namespace

__global__ void __launch_bounds__(OV_NT) overlap_kernel(OverlapParams p) {
  extern __shared__ uint32_t bms[];          // [N][OV_WWORDS]
  __shared__ int rng_lo[OVERLAP_MAX_N], rng_hi[OVERLAP_MAX_N], valid_n[OVERLAP_MAX_N], last_key[OVERLAP_MAX_N];
  const int tid = threadIdx.x;
  const int N = p.N;
  const int P = N * (N + 1) / 2;

  int pi[OV_PPT], pj[OV_PPT];
  unsigned long long acc[OV_PPT];
#pragma unroll
  for (int u = 0; u < OV_PPT; ++u) {
    acc[u] = 0ull;
    pi[u] = -1;
    pj[u] = -1;
    const int pp = tid + u * OV_NT;
    if (pp < P) {
      int i = 0, rem = pp;
      while (rem >= N - i) {
        rem -= N - i;
        ++i;
      }
      pi[u] = i;
      pj[u] = i + rem;
    }
  }

  const long long nrows = (p.row_end - p.row_begin + p.row_stride - 1) / p.row_stride;
  for (long long ri = blockIdx.x; ri < nrows; ri += gridDim.x) {
    const int t = (int)(p.row_begin + ri * p.row_stride);
    // number of valid (non-negative) entries of each layer's row: the -1
    // padding sits at the tail, so a binary search finds it
    if (tid < N) {
      const int32_t* row = p.idx[tid] + (size_t)t * p.topk;
      int lo = 0, hi = p.topk;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (row[mid] >= 0) lo = mid + 1;
        else hi = mid;
      }
      valid_n[tid] = lo;
      last_key[tid] = lo > 0 ? row[lo - 1] : -1;   // rows are ascending
    }
    __syncthreads();
    int kmax = -1;
    for (int i = 0; i < N; ++i) kmax = max(kmax, last_key[i]);
    kmax = min(kmax, OVERLAP_MAX_KEY);
    __syncthreads();   // every thread has read last_key before the next row rewrites it
    const int nwin = (kmax + OV_WBITS) / OV_WBITS;   // windows covering [0, kmax]
    for (int win = 0; win < nwin; ++win) {
      const int v0 = win * OV_WBITS;
      for (int i = tid; i < N * OV_WWORDS; i += OV_NT) bms[i] = 0u;
      if (tid < N) {
        const int32_t* row = p.idx[tid] + (size_t)t * p.topk;
        rng_lo[tid] = lower_bound_i32(row, valid_n[tid], v0);
        rng_hi[tid] = lower_bound_i32(row, valid_n[tid], v0 + OV_WBITS);
      }
      __syncthreads();
      for (int i = 0; i < N; ++i) {
        const int32_t* row = p.idx[i] + (size_t)t * p.topk;
        const int lo = rng_lo[i], hi = rng_hi[i];
        for (int e = lo + tid; e < hi; e += OV_NT) {
          const int v = row[e] - v0;
          if (v >= 0 && v < OV_WBITS) atomicOr(&bms[i * OV_WWORDS + (v >> 5)], 1u << (v & 31));
        }
      }
      __syncthreads();
      const int nwords = min(OV_WWORDS, (kmax + 1 - v0 + 31) >> 5);
#pragma unroll
      for (int u = 0; u < OV_PPT; ++u) {
        if (pi[u] >= 0) {
          const uint32_t* a = bms + pi[u] * OV_WWORDS;
          const uint32_t* c = bms + pj[u] * OV_WWORDS;
          unsigned s = 0;
          for (int wd = 0; wd < nwords; ++wd) s += __popc(a[wd] & c[wd]);
          acc[u] += s;
        }
      }
      __syncthreads();
    }
  }
#pragma unroll
  for (int u = 0; u < OV_PPT; ++u) {
    if (pi[u] >= 0 && acc[u]) {
      atomicAdd(&p.counts[pi[u] * N + pj[u]], acc[u]);
      if (pi[u] != pj[u]) atomicAdd(&p.counts[pj[u] * N + pi[u]], acc[u]);
    }
  }
}

__global__ void overlap_prepare_kernel(unsigned long long* counts, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) counts[i] = 0ull;
}

size_t overlap_lds_bytes(int N) { return (size_t)N * OV_WWORDS * sizeof(uint32_t); }

hipError_t overlap_launch(const OverlapParams& p, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(overlap_prepare_kernel, dim3(1), dim3(256), 0, stream, p.counts, p.N * p.N);
  hipLaunchKernelGGL(overlap_kernel, dim3(grid), dim3(OV_NT), overlap_lds_bytes(p.N), stream, p);
  return hipGetLastError();
}

}  // namespace dsa
