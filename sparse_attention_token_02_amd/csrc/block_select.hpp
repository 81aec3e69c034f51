// Workgroup-cooperative exact top-k of a candidate list.
//
// The list (score, key index) lives in global memory in ascending key-index
// order.  block_select keeps the k best entries under the total order
// "score descending, then key index ascending" and writes them, still in
// ascending key-index order, to the destination (which may be the list
// itself).  The k-th score is found by MSB-first radix select on the
// order-preserving 32-bit key of the score (digits start below the bits that
// all entries share); entries equal to that key are then taken in list order,
// i.e. lowest key index first.  Integer counting only, so the result does not
// depend on thread scheduling.
#pragma once
#include "device_common.hpp"

namespace dsa {

template <int NT>
struct SelectShared {
  uint32_t hist[256];
  uint32_t red[2][NT / 64];
  int wtot_eq[NT / 64];
  int wtot_keep[2][NT / 64];
  int bcast[2];
};

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
}

// Returns the number of entries written (min(k, cnt)).  If tau_out is not
// null, thread 0 stores the score of the k-th kept entry there (the smallest
// kept score) when cnt > k.  dsc may be null (scores not wanted).  Entries
// [written, pad_to) of the destination are set to (-inf, -1).
template <int NT>
__device__ int block_select(const float* sc, const int* ix, int cnt, int k, float* dsc, int* dix,
                            int pad_to, SelectShared<NT>& sh, float* tau_out) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  constexpr int NW = NT / 64;
  int written;
  if (cnt <= k) {
    if (dix != ix) {
      for (int j = tid; j < cnt; j += NT) {
        int x = ix[j];
        float s = sc[j];
        dix[j] = x;
        if (dsc) dsc[j] = s;
      }
    }
    written = cnt;
  } else {
    // ---- range of keys: skip the leading bits every entry shares
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
    for (int j = tid; j < cnt; j += NT) {
      uint32_t key = ordered_key(sc[j]);
      lo = min(lo, key);
      hi = max(hi, key);
    }
    lo = wave_min_u32(lo);
    hi = wave_max_u32(hi);
    if (lane == 0) {
      sh.red[0][wave] = lo;
      sh.red[1][wave] = hi;
    }
    __syncthreads();
    lo = 0xFFFFFFFFu;
    hi = 0u;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      lo = min(lo, sh.red[0][w]);
      hi = max(hi, sh.red[1][w]);
    }
    int need = k;
    uint32_t prefix = hi, pmask = 0xFFFFFFFFu;
    if (lo != hi) {
      const int top = 31 - __clz(lo ^ hi);
      pmask = (top == 31) ? 0u : (0xFFFFFFFFu << (top + 1));
      prefix = hi & pmask;
      for (int bit = top; bit >= 0;) {
        const int nb = bit + 1 < 8 ? bit + 1 : 8;
        const int shift = bit + 1 - nb;
        const uint32_t dm = (1u << nb) - 1u;
        for (int i = tid; i < 256; i += NT) sh.hist[i] = 0u;
        __syncthreads();
        for (int j = tid; j < cnt; j += NT) {
          uint32_t key = ordered_key(sc[j]);
          if ((key & pmask) == prefix) atomicAdd(&sh.hist[(key >> shift) & dm], 1u);
        }
        __syncthreads();
        if (wave == 0) {
          uint32_t h[4];
          uint32_t s = 0;
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            h[b] = sh.hist[4 * lane + b];
            s += h[b];
          }
          // inclusive suffix sum over lanes: sum of bins of this lane and all above
          uint32_t incl = s;
#pragma unroll
          for (int o = 1; o < 64; o <<= 1) {
            uint32_t t = (uint32_t)__shfl_down((int)incl, o);
            if (lane + o < 64) incl += t;
          }
          uint32_t cum = incl - s;
#pragma unroll
          for (int b = 3; b >= 0; --b) {
            if (cum < (uint32_t)need && cum + h[b] >= (uint32_t)need) {
              sh.bcast[0] = 4 * lane + b;
              sh.bcast[1] = (int)cum;
            }
            cum += h[b];
          }
        }
        __syncthreads();
        const uint32_t d = (uint32_t)sh.bcast[0];
        need -= sh.bcast[1];
        prefix |= d << shift;
        pmask |= dm << shift;
        bit -= nb;
        __syncthreads();
      }
    }
    const uint32_t kstar = prefix;
    // ---- stable compaction: keys above kstar, then the first `need` equal to it
    written = 0;
    int ties_seen = 0;
    int par = 0;
    for (int base = 0; base < cnt; base += NT, par ^= 1) {
      const int j = base + tid;
      const bool in = j < cnt;
      float s = 0.f;
      int x = 0;
      uint32_t key = 0u;
      if (in) {
        s = sc[j];
        x = ix[j];
        key = ordered_key(s);
      }
      const bool gt = in && key > kstar;
      const bool eq = in && key == kstar;
      const uint64_t beq = ballot64(eq);
      if (lane == 0) sh.wtot_eq[wave] = __popcll(beq);
      __syncthreads();
      int eq_pre = lanes_below(beq), eq_tot = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const int v = sh.wtot_eq[w];
        eq_pre += (w < wave) ? v : 0;
        eq_tot += v;
      }
      const bool keep = gt || (eq && ties_seen + eq_pre < need);
      const uint64_t bk = ballot64(keep);
      if (lane == 0) sh.wtot_keep[par][wave] = __popcll(bk);
      __syncthreads();
      int k_pre = lanes_below(bk), k_tot = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const int v = sh.wtot_keep[par][w];
        k_pre += (w < wave) ? v : 0;
        k_tot += v;
      }
      if (keep) {
        dix[written + k_pre] = x;
        if (dsc) dsc[written + k_pre] = s;
      }
      written += k_tot;
      ties_seen += eq_tot;
    }
    if (tau_out && tid == 0) *tau_out = key_to_float(kstar);
  }
  for (int j = written + tid; j < pad_to; j += NT) {
    dix[j] = -1;
    if (dsc) dsc[j] = -__builtin_inff();
  }
  __syncthreads();
  return written;
}

}  // namespace dsa
