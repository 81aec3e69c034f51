// Stand-in consumer of the decode selection for gfx950: single-head sparse
// softmax attention of one decode query per sequence over the k cache rows
// its layer attends ("Multi-layer Indexer", abstract: every DSA layer attends
// only the k = 2048 tokens an indexer selected).  It exists to give the
// layer schedules a consumer with the memory traffic of sparse MLA decode
// (each selected row is one 576-value bf16 latent vector, read once); it is
// not a model's attention layer.
//
//   s_j = scale * q[b] . latent[b, T_j, 0:576]
//   out[b, :] = sum_j softmax(s)_j * latent[b, T_j, 0:512]
//
// over the non-negative entries T_j of the selection row (-1 padding is
// skipped).  Two kernels: workgroups of 4 waves take 128 selection entries
// each (staged in LDS first, so row loads never wait on an index load), each
// wave keeps 8 rows in flight and a running (max, sum, weighted rows) with
// one online-softmax update per batch; a combine kernel merges the partials
// with their max offsets.
#include "device_common.hpp"
#include "kernels.hpp"

namespace dsa {

namespace {
constexpr int SA_NT = 256;
constexpr int SA_WAVES = SA_NT / 64;
constexpr int SA_U = 8;   // rows in flight per wave

// eight bf16 values (16 bytes) widened to fp32
__device__ __forceinline__ void widen8(uint4 v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

}  // namespace

__global__ void __launch_bounds__(SA_NT) standin_attn_partial_kernel(StandinAttnParams p) {
  const int b = blockIdx.y, split = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __shared__ int sidx[STANDIN_ROWS];
  __shared__ float wm[SA_WAVES], wl[SA_WAVES];
  __shared__ float wacc[SA_WAVES][STANDIN_DV];

  // this workgroup's selection entries, once; -1 marks padding and entries
  // outside the cache
  const int j0 = split * STANDIN_ROWS;
  for (int i = threadIdx.x; i < STANDIN_ROWS; i += SA_NT) {
    const int jj = j0 + i;
    int sv = jj < p.topk ? p.sel[(size_t)b * p.topk + jj] : -1;
    sidx[i] = sv < p.Lmax ? sv : -1;
  }

  // lane l holds dims 8l .. 8l+7 of the first 512 and, for l < 8, dims
  // 512+8l .. 512+8l+7 of the last 64; every lane holds value dims 8l .. 8l+7
  const uint4* qv = reinterpret_cast<const uint4*>(p.q + (size_t)b * STANDIN_DK);
  float qa[8], qb[8];
  widen8(qv[lane], qa);
  if (lane < 8) widen8(qv[64 + lane], qb);
  else
#pragma unroll
    for (int e = 0; e < 8; ++e) qb[e] = 0.f;
  __syncthreads();

  const uint16_t* base = p.latent + (size_t)b * p.Lmax * STANDIN_DK;
  float m = -__builtin_inff(), l = 0.f, acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;

  // wave w takes entries w*RPW .. w*RPW+RPW-1, SA_U rows per batch in flight
  constexpr int RPW = STANDIN_ROWS / SA_WAVES;
  static_assert(RPW % SA_U == 0, "whole batches per wave");
  for (int r0 = 0; r0 < RPW; r0 += SA_U) {
    int s[SA_U];
    uint4 va[SA_U], vb[SA_U];
#pragma unroll
    for (int u = 0; u < SA_U; ++u) {
      s[u] = sidx[wave * RPW + r0 + u];
      const uint4* row = reinterpret_cast<const uint4*>(base + (size_t)max(s[u], 0) * STANDIN_DK);
      va[u] = s[u] >= 0 ? row[lane] : make_uint4(0, 0, 0, 0);
      vb[u] = (s[u] >= 0 && lane < 8) ? row[64 + lane] : make_uint4(0, 0, 0, 0);
    }
    float d[SA_U], v[SA_U][8];
#pragma unroll
    for (int u = 0; u < SA_U; ++u) {
      float x[8];
      widen8(va[u], v[u]);
      widen8(vb[u], x);
      float t = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) t = fmaf(qa[e], v[u][e], fmaf(qb[e], x[e], t));
      d[u] = t;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
#pragma unroll
      for (int u = 0; u < SA_U; ++u) d[u] += __shfl_xor(d[u], o);
    // one online-softmax step for the batch (row validity is uniform)
    float bm = -__builtin_inff();
#pragma unroll
    for (int u = 0; u < SA_U; ++u) {
      d[u] = s[u] >= 0 ? p.scale * d[u] : -__builtin_inff();
      bm = fmaxf(bm, d[u]);
    }
    if (bm == -__builtin_inff()) continue;
    const float mn = fmaxf(m, bm);
    const float a = __expf(m - mn);   // 0 while m is still -inf
    l *= a;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= a;
#pragma unroll
    for (int u = 0; u < SA_U; ++u) {
      const float pu = __expf(d[u] - mn);   // 0 for a skipped row
      l += pu;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(pu, v[u][e], acc[e]);
    }
    m = mn;
  }
  if (lane == 0) {
    wm[wave] = m;
    wl[wave] = l;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) wacc[wave][8 * lane + e] = acc[e];
  __syncthreads();
  // merge the waves: partial = (max, sum, weighted rows) of this workgroup
  float* out = p.part + ((size_t)b * gridDim.x + split) * STANDIN_PART;
  float mm = -__builtin_inff();
#pragma unroll
  for (int w = 0; w < SA_WAVES; ++w) mm = fmaxf(mm, wm[w]);
  float f[SA_WAVES];
#pragma unroll
  for (int w = 0; w < SA_WAVES; ++w) f[w] = wm[w] == -__builtin_inff() ? 0.f : __expf(wm[w] - mm);
  for (int dd = threadIdx.x; dd < STANDIN_DV; dd += SA_NT) {
    float a = 0.f;
#pragma unroll
    for (int w = 0; w < SA_WAVES; ++w) a = fmaf(f[w], wacc[w][dd], a);
    out[4 + dd] = a;
  }
  if (threadIdx.x == 0) {
    float ls = 0.f;
#pragma unroll
    for (int w = 0; w < SA_WAVES; ++w) ls = fmaf(f[w], wl[w], ls);
    out[0] = mm;
    out[1] = ls;
  }
}

__global__ void __launch_bounds__(STANDIN_DV) standin_attn_combine_kernel(StandinAttnParams p, int splits) {
  const int b = blockIdx.x, d = threadIdx.x;
  const float* part = p.part + (size_t)b * splits * STANDIN_PART;
  float mm = -__builtin_inff();
  for (int i = 0; i < splits; ++i) mm = fmaxf(mm, part[(size_t)i * STANDIN_PART]);
  float ls = 0.f, a = 0.f;
  if (mm != -__builtin_inff()) {
    for (int i = 0; i < splits; ++i) {
      const float* q = part + (size_t)i * STANDIN_PART;
      if (q[0] == -__builtin_inff()) continue;
      const float f = __expf(q[0] - mm);
      ls = fmaf(f, q[1], ls);
      a = fmaf(f, q[4 + d], a);
    }
  }
  p.out[(size_t)b * STANDIN_DV + d] = ls > 0.f ? a / ls : 0.f;
}

int standin_attn_splits(int topk) { return (topk + STANDIN_ROWS - 1) / STANDIN_ROWS; }

hipError_t standin_attn_launch(const StandinAttnParams& p, hipStream_t stream) {
  const int splits = standin_attn_splits(p.topk);
  hipLaunchKernelGGL(standin_attn_partial_kernel, dim3(splits, p.B), dim3(SA_NT), 0, stream, p);
  hipLaunchKernelGGL(standin_attn_combine_kernel, dim3(p.B), dim3(STANDIN_DV), 0, stream, p, splits);
  return hipGetLastError();
}

}  // namespace dsa
