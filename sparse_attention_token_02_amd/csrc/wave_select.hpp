// Wave-level (64-lane) selection for gfx950: exact k-th largest key of a set
// of floats and exact top-k of a candidate list, each run by one wave with
// a 256-bin histogram in LDS and no workgroup barrier.  Everything is
// inlined: as called functions these took generic pointers, so the
// histogram updates became FLAT atomics and every call saved registers to
// scratch.
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
// With COPIES > 1 the histogram is COPIES interleaved partial counts, bin b
// copy c at word COPIES * b + c (summed here).
// Returns d such that the bins above d hold fewer than `need` entries and
// bins d and above hold at least `need` (requires 1 <= need <= total).
// *above = entries in bins above d, *count = entries in bin d.
template <int COPIES = 1>
__device__ __forceinline__ int wave_boundary_digit(const uint32_t* hist, uint32_t need, uint32_t* above,
                                                   uint32_t* count) {
  const int lane = __lane_id();
  uint32_t h[4], sum = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    h[b] = 0;
#pragma unroll
    for (int c = 0; c < COPIES; ++c) h[b] += hist[COPIES * (4 * lane + b) + c];
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

// Calls body(key) for the keys ordered_key(vals[i]), i < n, in no
// particular order.  vals is 16-byte aligned; a lane reads four consecutive
// entries per 16-byte load and issues eight loads (2048 entries per wave)
// before it uses any.  The float4 holding entry n - 1 is the last one read,
// so reads stay inside the 16-byte-rounded array.
template <class Body>
__device__ __forceinline__ void wave_for_score_keys(const float* vals, int n, Body body) {
  constexpr int U = 8;
  const int nq = (n + 3) >> 2;
  for (int q0 = __lane_id(); q0 < nq; q0 += 64 * U) {
    v4f v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = reinterpret_cast<const v4f*>(vals)[min(q0 + 64 * u, nq - 1)];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (q0 + 64 * u < nq)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (4 * (q0 + 64 * u) + e < n) body(ordered_key(v[u][e]));
  }
}

// Selection rule produced by the radix search: an entry with key K is kept
// if (K & mask) > prefix, or if (K & mask) == prefix and it is among the
// first `take_eq` such entries in list order.  kth is the k-th largest key.
struct WaveCut {
  uint32_t mask, prefix, take_eq, kth;
};

// Radix search for the cut that keeps exactly k of the n keys of vals[0..n)
// (requires n > k >= 1).  Stops as soon as the boundary bin is kept whole;
// the k-th key is then the smallest key of that bin, found with one more
// pass when need_kth (else kth is left 0).  `hist` is COPIES * 256 words of
// this wave's LDS: lane l counts into copy l % COPIES, the copies of a bin
// adjacent, so lanes that hit the same bin at once (scores sharing their
// leading bits) spread over COPIES addresses in different banks.  lo_hi,
// when given, holds the smallest and largest key (reduced over the wave),
// which saves the first pass.
template <int COPIES = 1>
__device__ __forceinline__ WaveCut wave_find_cut(const float* vals, int n, int k, uint32_t* hist, bool need_kth = true,
                                 const uint32_t* lo_hi = nullptr) {
  const int lane = __lane_id();
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
  if (lo_hi) {
    lo = lo_hi[0];
    hi = lo_hi[1];
  } else {
    wave_for_score_keys(vals, n, [&](uint32_t key) {
      lo = min(lo, key);
      hi = max(hi, key);
    });
  }
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
    for (int b = 0; b < 4 * COPIES; ++b) hist[64 * b + lane] = 0u;
    wave_lds_sync();
    wave_for_score_keys(vals, n, [&](uint32_t key) {
      if ((key & pmask) == prefix) atomicAdd(&hist[COPIES * ((key >> shift) & dm) + (lane & (COPIES - 1))], 1u);
    });
    wave_lds_sync();
    uint32_t above, count;
    const int d = wave_boundary_digit<COPIES>(hist, need, &above, &count);
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
  if (whole_bin && !need_kth) kth = 0u;
  if (whole_bin && need_kth) {
    // the k-th key is the smallest key of the boundary bin
    uint32_t m = 0xFFFFFFFFu;
    wave_for_score_keys(vals, n, [&](uint32_t key) {
      if ((key & pmask) == prefix) m = min(m, key);
    });
    kth = (uint32_t)__builtin_amdgcn_readfirstlane((int)wave_min_u32(m));
  }
  return WaveCut{pmask, prefix, need, kth};
}

// k-th largest key (1 <= kp <= n) among the n floats vals[0..n) (16-byte aligned).
__device__ __forceinline__ uint32_t wave_kth_key(const float* vals, int n, int kp, uint32_t* hist) {
  if (n == 1) return ordered_key(vals[0]);
  if (kp >= n) {
    uint32_t lo = 0xFFFFFFFFu;
    wave_for_score_keys(vals, n, [&](uint32_t key) { lo = min(lo, key); });
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)wave_min_u32(lo));
  }
  return wave_find_cut(vals, n, kp, hist).kth;
}

// Exact top-k of the candidate list (sc[i], ix[i]), i < n, held in global
// memory in ascending key-index order (both arrays 16-byte aligned).  Keeps
// the k largest scores, ties to the earliest entries, and writes the kept
// entries in list order to dix[0..) and dsc[0..) (dsc may be null; dix/dsc
// may alias ix/sc: a batch is read whole before any of it is written, and
// writes never pass the start of the next batch).  Then pads dix with -1 and
// dsc with -inf up to pad_to.  Returns the number kept, min(n, k).  *tau (if
// not null) receives the k-th largest score (-inf when n <= k).
// The caller makes the list's earlier global writes visible first.
// lbuf (16-byte aligned wave-private LDS of lcap floats, lcap a multiple of
// 4, or null): when the list fits, its scores are copied there once and every
// later pass reads them from LDS (then dsc must not alias sc).
// hist: COPIES * 256 words (see wave_find_cut).
// STREAM_OUT: the output is final (not read again by this kernel): written
// with non-temporal stores, so it does not stay behind as dirty cache lines.
// When lbuf can hold the min(n, k) kept indices, they are gathered there
// first (at their output positions, all of which precede the entries still
// to be read) and written out with whole-line stores at the end; scattered
// non-temporal stores would reach HBM as partial lines, several per line.
template <int COPIES = 1, bool STREAM_OUT = false>
__device__ __forceinline__ int wave_select(const float* sc, const int* ix, int n, int k, float* dsc, int* dix, int pad_to,
                           uint32_t* hist, float* tau, float* lbuf = nullptr, int lcap = 0) {
  const int lane = __lane_id();
  WaveCut cut{0u, 0u, 0xFFFFFFFFu, 0u};   // keeps everything
  const float* ksc = sc;                  // where the scores are read from
  uint32_t lo_hi[2];
  bool have_lo_hi = false;
  if (lbuf && n > k && n <= lcap) {
    // copy the scores, rounded up to whole float4 groups (inside the list's
    // 16-byte-rounded storage and inside lcap), eight loads in flight per
    // lane, and take the smallest and largest key on the way
    constexpr int UC = 8;
    const int nq = (n + 3) >> 2;
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
    for (int q0 = lane; q0 < nq; q0 += 64 * UC) {
      v4f v[UC];
#pragma unroll
      for (int u = 0; u < UC; ++u) v[u] = reinterpret_cast<const v4f*>(sc)[min(q0 + 64 * u, nq - 1)];
#pragma unroll
      for (int u = 0; u < UC; ++u)
        if (q0 + 64 * u < nq) {
          reinterpret_cast<v4f*>(lbuf)[q0 + 64 * u] = v[u];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (4 * (q0 + 64 * u) + e < n) {
              const uint32_t key = ordered_key(v[u][e]);
              lo = min(lo, key);
              hi = max(hi, key);
            }
        }
    }
    lo_hi[0] = (uint32_t)__builtin_amdgcn_readfirstlane((int)wave_min_u32(lo));
    lo_hi[1] = (uint32_t)__builtin_amdgcn_readfirstlane((int)wave_max_u32(hi));
    have_lo_hi = true;
    wave_lds_sync();
    ksc = lbuf;
  }
  if (n > k) cut = wave_find_cut<COPIES>(ksc, n, k, hist, tau != nullptr, have_lo_hi ? lo_hi : nullptr);
  if (tau) *tau = n > k ? key_to_float(cut.kth) : -__builtin_inff();
  int* ob = nullptr;                      // staged output indices (STREAM_OUT)
  if constexpr (STREAM_OUT)
    if (lbuf && min(n, k) <= lcap) ob = reinterpret_cast<int*>(lbuf);
  int out = 0;
  uint32_t eq_seen = 0;
  constexpr int U = 4;                    // float4 groups per lane and batch
  const int nq = (n + 3) >> 2;
  for (int q0 = 0; q0 < nq; q0 += 64 * U) {
    // the batch: entries 4 (q0 + 64 u + lane) + e, read whole before any write
    v4f sv[U];
    v4i iv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int q = min(q0 + 64 * u + lane, nq - 1);
      sv[u] = reinterpret_cast<const v4f*>(ksc)[q];
      iv[u] = reinterpret_cast<const v4i*>(ix)[q];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e0 = 4 * (q0 + 64 * u + lane);
      uint32_t gt = 0, eq = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool valid = e0 + e < n;
        const uint32_t km = ordered_key(sv[u][e]) & cut.mask;
        gt |= (uint32_t)(valid && km > cut.prefix) << e;
        eq |= (uint32_t)(valid && km == cut.prefix) << e;
      }
      // ties are taken in list order: rank = ties before this lane + within
      // it.  One scan carries both counts: ties in the low 16 bits, kept
      // entries above the cut in the high 16 (each at most 256 per wave)
      const int neq = __popc(eq);
      const int ngt = __popc(gt);
      const int both_incl = wave_incl_sum(neq | (ngt << 16));
      const int eq_incl = both_incl & 0xFFFF;
      uint32_t rank = eq_seen + (uint32_t)(eq_incl - neq);
      uint32_t take = gt;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if ((eq >> e) & 1u) {
          if (rank < cut.take_eq) take |= 1u << e;
          ++rank;
        }
      // kept ties of this lane and of the lanes before it: the ties before
      // this lane that are still below take_eq, plus this lane's own
      const int eq_before = eq_incl - neq;
      const uint32_t room_u = cut.take_eq > eq_seen ? cut.take_eq - eq_seen : 0u;   // ties still to take
      const int room = (int)min(room_u, 0x7FFFFFFFu);
      const int teq_before = min(eq_before, room);
      const int teq_incl = min(eq_incl, room);
      const int nt_incl = (both_incl >> 16) + teq_incl;
      int pos = out + (both_incl >> 16) - ngt + teq_before;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if ((take >> e) & 1u) {
          if constexpr (STREAM_OUT) {
            if (ob) ob[pos] = iv[u][e];
            else __builtin_nontemporal_store(iv[u][e], dix + pos);
            if (dsc) __builtin_nontemporal_store(sv[u][e], dsc + pos);
          } else {
            dix[pos] = iv[u][e];
            if (dsc) dsc[pos] = sv[u][e];
          }
          ++pos;
        }
      out += __builtin_amdgcn_readlane(nt_incl, 63);
      eq_seen += (uint32_t)__builtin_amdgcn_readlane(eq_incl, 63);
    }
  }
  if constexpr (STREAM_OUT) {
    if (ob) {
      // the row from the 256-byte boundary at or below dix: each store
      // instruction covers one aligned 256-byte block
      wave_lds_sync();
      const int b0 = -(int)((reinterpret_cast<uintptr_t>(dix) >> 2) & 63);
      for (int e = b0 + lane; e < pad_to; e += 64)
        if (e >= 0) __builtin_nontemporal_store(e < out ? ob[e] : -1, dix + e);
    }
  }
  for (int e = out + lane; e < pad_to; e += 64) {
    if constexpr (STREAM_OUT) {
      if (!ob) __builtin_nontemporal_store(-1, dix + e);
      if (dsc) __builtin_nontemporal_store(-__builtin_inff(), dsc + e);
    } else {
      dix[e] = -1;
      if (dsc) dsc[e] = -__builtin_inff();
    }
  }
  return out;
}

}  // namespace dsa
