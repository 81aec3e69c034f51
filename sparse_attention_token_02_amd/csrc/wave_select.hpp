// Wave-level (64-lane) selection for gfx950: exact k-th largest key of a set
// of floats and exact top-k of a candidate list, each run by one wave with
// a 256-bin histogram in LDS and no workgroup barrier.
//
// Keys: order-preserving 32-bit images of the scores (ordered_key), so a
// radix select over key bits, most significant first, finds the k-th score
// exactly.  Ties are broken by list position (earliest first), which for a
// list kept in ascending key-index order is "lowest index wins" (IndexCache
// deep-dive report, section 1.1: the indexer keeps the k best keys per query).
#pragma once
#include "device_common.hpp"

namespace dsa {

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

// Boundary digit of a 256-bin histogram whose bins are indexed by digit
// value (larger digit = larger key), 4 bins per lane (lane l: 4l..4l+3).
// Returns d such that the bins above d hold fewer than `need` entries and
// bins d and above hold at least `need` (requires 1 <= need <= total).
// *above = entries in bins above d, *count = entries in bin d.
__device__ __forceinline__ int wave_boundary_digit(const uint32_t* hist, uint32_t need, uint32_t* above,
                                                   uint32_t* count) {
  const int lane = __lane_id();
  uint32_t h[4], sum = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    h[b] = hist[4 * lane + b];
    sum += h[b];
  }
  // entries in the bins of this lane and all higher lanes
  uint32_t incl = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = (uint32_t)__shfl_down((int)incl, o);
    if (lane + o < 64) incl += t;
  }
  uint32_t cum = incl - sum;
  int dig = -1;
  uint32_t ab = 0, cnt = 0;
#pragma unroll
  for (int b = 3; b >= 0; --b) {
    if (cum < need && cum + h[b] >= need) {
      dig = 4 * lane + b;
      ab = cum;
      cnt = h[b];
    }
    cum += h[b];
  }
  const uint64_t who = ballot64(dig >= 0);
  const int src = __ffsll((long long)who) - 1;
  *above = (uint32_t)__builtin_amdgcn_readlane((int)ab, src);
  *count = (uint32_t)__builtin_amdgcn_readlane((int)cnt, src);
  return __builtin_amdgcn_readlane(dig, src);
}

// Calls body(key) for key_of(i), i < n, over this lane's entries (i = lane
// + 64 j).  Keys are fetched eight at a time (indices clamped into range, so
// the loads are unconditional) before any is used, which keeps eight memory
// reads in flight per lane.
template <class KeyOf, class Body>
__device__ __forceinline__ void wave_for_keys(KeyOf key_of, int n, Body body) {
  constexpr int U = 8;
  for (int base = __lane_id(); base < n; base += 64 * U) {
    uint32_t kk[U];
#pragma unroll
    for (int u = 0; u < U; ++u) kk[u] = key_of(min(base + 64 * u, n - 1));
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (base + 64 * u < n) body(kk[u]);
  }
}

// Selection rule produced by the radix search: an entry with key K is kept
// if (K & mask) > prefix, or if (K & mask) == prefix and it is among the
// first `take_eq` such entries in list order.  kth is the k-th largest key.
struct WaveCut {
  uint32_t mask, prefix, take_eq, kth;
};

// Radix search for the cut that keeps exactly k of the n keys key_of(i),
// i < n (requires n > k >= 1).  Stops as soon as the boundary bin is kept
// whole; the k-th key is then the smallest key of that bin (one more pass).
// `hist` is 256 words of this wave's LDS.
template <class KeyOf>
__device__ WaveCut wave_find_cut(KeyOf key_of, int n, int k, uint32_t* hist) {
  const int lane = __lane_id();
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
  wave_for_keys(key_of, n, [&](uint32_t key) {
    lo = min(lo, key);
    hi = max(hi, key);
  });
  // Every lane holds the same reduced values; readfirstlane makes that
  // visible to the compiler so the radix loop below is scalar control flow.
  lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)wave_min_u32(lo));
  hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)wave_max_u32(hi));
  if (lo == hi) return WaveCut{0xFFFFFFFFu, hi, (uint32_t)k, hi};
  const int top = 31 - __clz((int)(lo ^ hi));
  uint32_t pmask = (top == 31) ? 0u : (0xFFFFFFFFu << (top + 1));
  uint32_t prefix = hi & pmask;
  uint32_t need = (uint32_t)k;
  bool whole_bin = false;
  for (int bit = top; bit >= 0;) {
    const int nb = bit + 1 < 8 ? bit + 1 : 8;
    const int shift = bit + 1 - nb;
    const uint32_t dm = (1u << nb) - 1u;
#pragma unroll
    for (int b = 0; b < 4; ++b) hist[4 * lane + b] = 0u;
    wave_lds_sync();
    wave_for_keys(key_of, n, [&](uint32_t key) {
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & dm], 1u);
    });
    wave_lds_sync();
    uint32_t above, count;
    const int d = wave_boundary_digit(hist, need, &above, &count);
    wave_lds_sync();   // every lane has read the histogram before it is cleared again
    need -= above;
    prefix |= (uint32_t)d << shift;
    pmask |= dm << shift;
    bit -= nb;
    if (count == need && bit >= 0) {   // every entry of the boundary bin is kept
      whole_bin = true;
      break;
    }
  }
  uint32_t kth = prefix;   // exact when every bit was resolved
  if (whole_bin) {
    // the k-th key is the smallest key of the boundary bin
    uint32_t m = 0xFFFFFFFFu;
    wave_for_keys(key_of, n, [&](uint32_t key) {
      if ((key & pmask) == prefix) m = min(m, key);
    });
    kth = (uint32_t)__builtin_amdgcn_readfirstlane((int)wave_min_u32(m));
  }
  return WaveCut{pmask, prefix, need, kth};
}

// k-th largest key (1 <= kp <= n) among the n floats vals[0..n).
__device__ __forceinline__ uint32_t wave_kth_key(const float* vals, int n, int kp, uint32_t* hist) {
  if (n == 1) return ordered_key(vals[0]);
  if (kp >= n) {
    uint32_t lo = 0xFFFFFFFFu;
    for (int e = __lane_id(); e < n; e += 64) lo = min(lo, ordered_key(vals[e]));
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)wave_min_u32(lo));
  }
  return wave_find_cut([&](int e) { return ordered_key(vals[e]); }, n, kp, hist).kth;
}

// Exact top-k of the candidate list (sc[i], ix[i]), i < n, held in global
// memory in ascending key-index order.  Keeps the k largest scores, ties to
// the earliest entries, and writes the kept entries in list order to
// dix[0..) and dsc[0..) (dsc may be null; dix/dsc may alias ix/sc, since an
// entry never moves to a later position).  Then pads dix with -1 and dsc with
// -inf up to pad_to.  Returns the number kept, min(n, k).  *tau (if not null)
// receives the k-th largest score (-inf when n <= k).
// The caller makes the list's earlier global writes visible first.
__device__ int wave_select(const float* sc, const int* ix, int n, int k, float* dsc, int* dix, int pad_to,
                           uint32_t* hist, float* tau) {
  const int lane = __lane_id();
  WaveCut cut{0u, 0u, 0xFFFFFFFFu, 0u};   // keeps everything
  if (n > k) cut = wave_find_cut([&](int e) { return ordered_key(sc[e]); }, n, k, hist);
  if (tau) *tau = n > k ? key_to_float(cut.kth) : -__builtin_inff();
  int out = 0;
  uint32_t eq_seen = 0;
  constexpr int U = 8;
  for (int base = 0; base < n; base += 64 * U) {
    // fetch eight groups of 64 entries, then emit them group by group in
    // list order (a group only writes below its own positions, so the
    // in-place case never overwrites an entry that is still to be read)
    float sv[U];
    int iv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = min(base + 64 * u + lane, n - 1);
      sv[u] = sc[e];
      iv[u] = ix[e];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool valid = base + 64 * u + lane < n;
      const uint32_t km = ordered_key(sv[u]) & cut.mask;
      const bool gt = valid && km > cut.prefix;
      const bool eq = valid && km == cut.prefix;
      const uint64_t meq = ballot64(eq);
      const bool take = gt || (eq && eq_seen + (uint32_t)lanes_below(meq) < cut.take_eq);
      const uint64_t mt = ballot64(take);
      if (take) {
        const int pos = out + lanes_below(mt);
        dix[pos] = iv[u];
        if (dsc) dsc[pos] = sv[u];
      }
      out += __popcll(mt);
      eq_seen += (uint32_t)__popcll(meq);
    }
  }
  for (int e = out + lane; e < pad_to; e += 64) {
    dix[e] = -1;
    if (dsc) dsc[e] = -__builtin_inff();
  }
  return out;
}

}  // namespace dsa
