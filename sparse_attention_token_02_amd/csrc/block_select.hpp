// Workgroup-cooperative exact top-k of a candidate list.
//
// The list (score, key index) lives in global memory in ascending key-index
// order.  block_select keeps the k best entries under the total order
// "score descending, then key index ascending" and writes them, still in
// ascending key-index order, to the destination (which may be the list
// itself).
//
// The list is first copied into LDS with 16-byte loads.  The k-th score is
// then found by MSB-first radix select on the order-preserving 32-bit key of
// the score: the digits start below the bits every entry shares, and once the
// boundary bin is small its entries are gathered into a short side list so
// later digits only touch those.  Entries equal to the k-th key are taken in
// list order, i.e. lowest key index first.  The result is written by a stable
// in-order pass.  Integer counting only: the output does not depend on thread
// scheduling.
#pragma once
#include "device_common.hpp"

namespace dsa {

constexpr int SEL_SIDE = 2048;   // side-list capacity (keys of the boundary bin)

template <int NT>
struct SelectShared {
  uint32_t hist[256];
  uint32_t red[2][NT / 64];
  int wtot_eq[NT / 64];
  int wtot_keep[NT / 64];
  int bcast[2];
  int side_n;
  uint32_t side[SEL_SIDE];
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

// Finds the digit d of the boundary bin from a 256-bin histogram: bins above d
// hold fewer than `need` entries, bins from d up hold at least `need`.
// Wave 0 scans; the result lands in sh.bcast = {d, count above d}.
template <int NT>
__device__ __forceinline__ void find_boundary(SelectShared<NT>& sh, int need) {
  const int lane = threadIdx.x & 63;
  if ((threadIdx.x >> 6) == 0) {
    uint32_t h[4];
    uint32_t s = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      h[b] = sh.hist[4 * lane + b];
      s += h[b];
    }
    uint32_t incl = s;   // suffix sum over lanes (this lane and above)
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t t = (uint32_t)__shfl_down((int)incl, o);
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
}

// Copies cnt (score, index) pairs from global memory into LDS.
template <int NT>
__device__ __forceinline__ void stage_list(const float* sc, const int* ix, int cnt, float* lsc, int* lix) {
  const int tid = threadIdx.x;
  const int n4 = cnt >> 2;
  for (int i = tid; i < n4; i += 2 * NT) {
    const int i2 = i + NT;
    const v4i a = reinterpret_cast<const v4i*>(sc)[i];
    const v4i b = reinterpret_cast<const v4i*>(ix)[i];
    v4i c = v4i{0, 0, 0, 0}, d = v4i{0, 0, 0, 0};
    if (i2 < n4) {
      c = reinterpret_cast<const v4i*>(sc)[i2];
      d = reinterpret_cast<const v4i*>(ix)[i2];
    }
    reinterpret_cast<v4i*>(lsc)[i] = a;
    reinterpret_cast<v4i*>(lix)[i] = b;
    if (i2 < n4) {
      reinterpret_cast<v4i*>(lsc)[i2] = c;
      reinterpret_cast<v4i*>(lix)[i2] = d;
    }
  }
  for (int j = 4 * n4 + tid; j < cnt; j += NT) {
    lsc[j] = sc[j];
    lix[j] = ix[j];
  }
}

// Keeps the k best of the list; see the file comment.  sc/ix: global list
// (16-byte aligned); lsc/lix: LDS scratch of at least cnt entries.  dsc may
// be null.  Entries [written, pad_to) of the destination become (-inf, -1).
// Returns min(k, cnt); thread 0 stores the k-th kept score in *tau_out when
// cnt > k and tau_out is not null.
template <int NT>
__device__ int block_select(const float* sc, const int* ix, int cnt, int k, float* dsc, int* dix, int pad_to,
                            SelectShared<NT>& sh, float* lsc, int* lix, float* tau_out) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  constexpr int NW = NT / 64;
  int written;
  if (cnt <= k) {
    if (dix != ix) {
      for (int j = tid; j < cnt; j += NT) {
        dix[j] = ix[j];
        if (dsc) dsc[j] = sc[j];
      }
    }
    written = cnt;
  } else {
    stage_list<NT>(sc, ix, cnt, lsc, lix);
    __syncthreads();
    // ---- range of keys: skip the leading bits every entry shares
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
    for (int j = tid; j < cnt; j += NT) {
      const uint32_t key = ordered_key(lsc[j]);
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
      bool on_side = false;
      int side_n = 0;
      for (int bit = top; bit >= 0;) {
        const int nb = bit + 1 < 8 ? bit + 1 : 8;
        const int shift = bit + 1 - nb;
        const uint32_t dm = (1u << nb) - 1u;
        for (int i = tid; i < 256; i += NT) sh.hist[i] = 0u;
        __syncthreads();
        if (on_side) {
          for (int j = tid; j < side_n; j += NT) {
            const uint32_t key = sh.side[j];
            if ((key & pmask) == prefix) atomicAdd(&sh.hist[(key >> shift) & dm], 1u);
          }
        } else {
          for (int j = tid; j < cnt; j += NT) {
            const uint32_t key = ordered_key(lsc[j]);
            if ((key & pmask) == prefix) atomicAdd(&sh.hist[(key >> shift) & dm], 1u);
          }
        }
        __syncthreads();
        find_boundary<NT>(sh, need);
        if (tid == 0) sh.side_n = 0;
        __syncthreads();
        const uint32_t d = (uint32_t)sh.bcast[0];
        const uint32_t bin_n = sh.hist[d];
        need -= sh.bcast[1];
        prefix |= d << shift;
        pmask |= dm << shift;
        bit -= nb;
        if (bit >= 0 && !on_side && bin_n <= (uint32_t)SEL_SIDE) {
          // gather the boundary bin's keys into the side list
          for (int j = tid; j < cnt; j += NT) {
            const uint32_t key = ordered_key(lsc[j]);
            if ((key & pmask) == prefix) sh.side[atomicAdd(&sh.side_n, 1)] = key;
          }
          on_side = true;
          side_n = (int)bin_n;
        }
        __syncthreads();
      }
    }
    const uint32_t kstar = prefix;
    // ---- stable compaction: keys above kstar, then the first `need` equal to it
    written = 0;
    int ties_seen = 0;
    for (int base = 0; base < cnt; base += NT) {
      const int j = base + tid;
      const bool in = j < cnt;
      float s = 0.f;
      int x = 0;
      uint32_t key = 0u;
      if (in) {
        s = lsc[j];
        x = lix[j];
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
      if (lane == 0) sh.wtot_keep[wave] = __popcll(bk);
      __syncthreads();
      int k_pre = lanes_below(bk), k_tot = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const int v = sh.wtot_keep[w];
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
