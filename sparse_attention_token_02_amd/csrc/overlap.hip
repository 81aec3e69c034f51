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
// keys; for each window every layer's keys are set in an LDS bitmap, then
// every thread ANDs and popcounts the bitmaps of its layer pairs (16 bytes
// per read) and keeps the running counts in registers until the workgroup is
// done.  The boundaries of each sorted list between windows are found up
// front, all at once (or, for rows of very many windows, one search per
// layer and window, each window starting where the previous one ended); each wave fills the bitmaps of its own layers, four at a time
// with 16 loads per lane and layer in flight.  Bitmap rows are padded so that consecutive layers start 4
// banks apart: lanes reading the same word of different layers do not
// collide.
#include "device_common.hpp"
#include "kernels.hpp"

namespace dsa {

namespace {
constexpr int OV_NT = 256;
constexpr int OV_WBITS = 8192;
constexpr int OV_WWORDS = OV_WBITS / 32;
constexpr int OV_RS = OV_WWORDS + 4;   // LDS words per layer bitmap row (16-byte aligned, 4 banks apart)
constexpr int OV_U = 16;               // index loads per lane and layer in one fill batch
constexpr int OV_G = 4;                // layers a wave fills together
constexpr int OV_MAXW = 16;            // rows of at most this many windows get all boundaries up front
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
  extern __shared__ __attribute__((aligned(16))) uint32_t bms[];   // [N][OV_RS]
  __shared__ int rng_lo[OVERLAP_MAX_N], rng_hi[OVERLAP_MAX_N], valid_n[OVERLAP_MAX_N], last_key[OVERLAP_MAX_N];
  __shared__ int bnd[OVERLAP_MAX_N][OV_MAXW + 1];   // bnd[i][w]: first entry of layer i in window w
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
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
    // padding sits at the tail, so a binary search finds it (a full row
    // needs only its last entry)
    if (tid < N) {
      const int32_t* row = p.idx[tid] + (size_t)t * p.topk;
      int lo = 0, hi = p.topk;
      if (row[p.topk - 1] >= 0) lo = p.topk;
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
    // Up to OV_MAXW windows: every boundary of every layer at once, as
    // independent searches spread over the workgroup (read after the first
    // window's barrier).  Longer rows search one boundary per window.
    const bool pre = nwin <= OV_MAXW;
    if (pre) {
      for (int q = tid; q < N * (nwin - 1); q += OV_NT) {
        const int i = q / (nwin - 1), w = 1 + q % (nwin - 1);
        bnd[i][w] = lower_bound_i32(p.idx[i] + (size_t)t * p.topk, valid_n[i], w * OV_WBITS);
      }
      if (tid < N) {
        bnd[tid][0] = 0;
        bnd[tid][nwin] = valid_n[tid];
      }
    }
    for (int win = 0; win < nwin; ++win) {
      const int v0 = win * OV_WBITS;
      for (int i = tid; i < N * OV_RS / 4; i += OV_NT) reinterpret_cast<v4i*>(bms)[i] = v4i{0, 0, 0, 0};
      if (!pre && tid < N) {   // each thread owns its layer's entry: no race with the previous window
        const int32_t* row = p.idx[tid] + (size_t)t * p.topk;
        rng_lo[tid] = win == 0 ? 0 : rng_hi[tid];
        rng_hi[tid] = lower_bound_i32(row, valid_n[tid], v0 + OV_WBITS);
      }
      __syncthreads();
      // wave w fills layers w, w + 4, ..., OV_G of them at a time, so that
      // OV_G * OV_U index loads per lane are in flight together
      constexpr int NW = OV_NT / 64;
      for (int i0 = wave; i0 < N; i0 += OV_G * NW) {
        const int32_t* row[OV_G];
        int lo[OV_G], hi[OV_G];
        int nb = 0;   // batches of the group's longest range (wave-uniform)
#pragma unroll
        for (int g = 0; g < OV_G; ++g) {
          const int i = i0 + g * NW;
          row[g] = p.idx[i < N ? i : 0] + (size_t)t * p.topk;
          lo[g] = i < N ? (pre ? bnd[i][win] : rng_lo[i]) : 0;
          hi[g] = i < N ? (pre ? bnd[i][win + 1] : rng_hi[i]) : 0;
          nb = max(nb, (hi[g] - lo[g] + 64 * OV_U - 1) / (64 * OV_U));
        }
        for (int bt = 0; bt < nb; ++bt) {
          int v[OV_G][OV_U];
#pragma unroll
          for (int g = 0; g < OV_G; ++g)
#pragma unroll
            for (int u = 0; u < OV_U; ++u)   // clamped into [0, hi): in bounds, unused past hi
              v[g][u] = row[g][max(min(lo[g] + 64 * (bt * OV_U + u) + lane, hi[g] - 1), 0)];
#pragma unroll
          for (int g = 0; g < OV_G; ++g)
#pragma unroll
            for (int u = 0; u < OV_U; ++u) {
              const int x = v[g][u] - v0;
              if (lo[g] + 64 * (bt * OV_U + u) + lane < hi[g] && x >= 0 && x < OV_WBITS)
                atomicOr(&bms[(i0 + g * NW) * OV_RS + (x >> 5)], 1u << (x & 31));
            }
        }
      }
      __syncthreads();
      const int nwords = min(OV_WWORDS, (kmax + 1 - v0 + 31) >> 5);
#pragma unroll
      for (int u = 0; u < OV_PPT; ++u) {
        if (pi[u] >= 0) {
          // whole 16-byte groups: words past nwords hold keys above every
          // layer's largest and are zero
          const v4i* a = reinterpret_cast<const v4i*>(bms + pi[u] * OV_RS);
          const v4i* c = reinterpret_cast<const v4i*>(bms + pj[u] * OV_RS);
          unsigned s = 0;
          for (int q = 0; q < (nwords + 3) >> 2; ++q) {
            const v4i x = a[q], y = c[q];
            s += __popc((uint32_t)(x[0] & y[0])) + __popc((uint32_t)(x[1] & y[1])) + __popc((uint32_t)(x[2] & y[2])) +
                 __popc((uint32_t)(x[3] & y[3]));
          }
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

size_t overlap_lds_bytes(int N) { return (size_t)N * OV_RS * sizeof(uint32_t); }

// Workgroups of the overlap kernel resident on one CU with N layers (at least
// 1): the grid is sized to this times the CU count, so that no workgroup
// waits for a second pass that would run with fewer neighbours to hide its
// load latency.
int overlap_blocks_per_cu(int N) {
  const size_t lds = overlap_lds_bytes(N);
  const void* fn = reinterpret_cast<const void*>(&overlap_kernel);
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess) return 1;
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, OV_NT, lds) != hipSuccess || nb < 1) return 1;
  return nb;
}

hipError_t overlap_launch(const OverlapParams& p, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(overlap_prepare_kernel, dim3(1), dim3(256), 0, stream, p.counts, p.N * p.N);
  const size_t lds = overlap_lds_bytes(p.N);   // above 64 KB for N = 64
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&overlap_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(overlap_kernel, dim3(grid), dim3(OV_NT), lds, stream, p);
  return hipGetLastError();
}

}  // namespace dsa
