// Fused prefill lightning indexer + streaming top-k for gfx950.
//
// What is computed (IndexCache deep-dive report, abstract and section 1.1:
// a multi-head ReLU-gated dot product, run in FP8, that scores every earlier
// token and keeps the k best):
//   score(t, s) = k_scale[s] * sum_h w[t,h] * q_scale[t,h] * ReLU(q[t,h] . k[s]),  s <= t
// and, per query row t, the min(k, t+1) best keys under "score descending,
// key index ascending", written in ascending key order and padded with -1.
//
// Design (one work item = RW consecutive query rows, 8 waves):
// * Score contraction on MFMA.  Index heads sit on the MFMA row dimension, so
//   the head sum stays inside a lane: with the 32x32 accumulator layout a lane
//   owns one key column and 16 rows, and the rows are assigned so that all 16
//   belong to one query (H >= 16) or to two queries of 8 heads (H == 8).  The
//   two lane halves therefore hold two different queries: no cross-lane
//   reduction at all.  Keys are the MFMA column dimension.
//   fp8 path: v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3 x e4m3, unit block
//   scales); bf16 path: v_mfma_f32_32x32x16_bf16.  Products are exact, the
//   accumulation is fp32.
// * Keys are staged through LDS in tiles of 64, double buffered; every wave
//   reuses each tile for its own queries.  Query operands and the folded head
//   weights w*q_scale stay in registers for the whole work item.
// * Epilogue per (query, key): sum_h w_eff * max(x, 0), times k_scale, causal
//   mask.  The L x L score matrix is never stored (the optional dense output
//   exists for small debugging runs only).
// * Streaming top-k: each row keeps a threshold tau (the current k-th best
//   score) and appends keys with score > tau, in ascending key order, to a
//   candidate list in the per-workgroup workspace.  Keys arrive in ascending
//   index order, so a later key that ties the k-th score always loses the tie
//   and "strictly greater" is the exact filter.  When a list could overflow
//   during the next tile, the whole workgroup compacts it to exactly k
//   entries (block_select), which also raises tau.  At the end of the work
//   item the same routine selects the final k and writes them out in order.
// * Persistent grid: one workgroup per CU pulls work items from an atomic
//   counter, longest (highest t) first, which balances the causal triangle.
#include "device_common.hpp"
#include "block_select.hpp"
#include "kernels.hpp"

namespace dsa {

namespace {

constexpr int NT = 512;      // threads per workgroup (8 waves)
constexpr int WAVES = NT / 64;
constexpr int TK = 128;      // keys per LDS tile

template <int DT, int H, int D>
struct PfCfg {
  static constexpr bool FP8 = (DT == DSA_FP8_E4M3);
  static constexpr int HB = H < 16 ? H : 16;        // heads of one query in one lane-block
  static constexpr int QPH = 16 / HB;               // queries per lane half
  static constexpr int QPW = 2 * QPH;               // queries per wave
  static constexpr int MB = H < 16 ? 1 : H / 16;    // 32-row MFMA blocks per wave
  static constexpr int ESZ = FP8 ? 1 : 2;           // bytes per element
  static constexpr int KM = FP8 ? 64 : 16;          // K of one MFMA
  static constexpr int KS = D / KM;                 // MFMAs along D
  static constexpr int SB = FP8 ? 32 : 16;          // bytes per lane per MFMA operand
  static constexpr int ROWB = D * ESZ;              // bytes of one key / one query head
  static constexpr int RW = WAVES * QPW;            // query rows per work item
  static constexpr int STRIDE = ROWB + 16;          // padded LDS row (bank-conflict free b128 reads)
  static constexpr int CHUNKS = TK * ROWB / 16;     // 16-byte pieces of a key tile
  static constexpr int CPT = (CHUNKS + NT - 1) / NT;
  static_assert(H == 8 || (H % 16 == 0 && H <= 64), "unsupported head count");
  static_assert(D % KM == 0 && ROWB / 2 == KS * SB, "unsupported head dim");
  static_assert(RW <= 32, "row mask is 32 bits");
};

template <int DT, int H, int D>
struct PfShared {
  using C = PfCfg<DT, H, D>;
  uint8_t ktile[2][TK * C::STRIDE];     // double-buffered key tile
  float kscale[2][TK];
  float stage_sc[C::RW][TK];            // this tile's accepted candidates, per row
  int stage_ix[C::RW][TK];
  SelectShared<NT> sel;
  uint32_t whist[WAVES][256];           // per-wave histogram for the sample quantile
  int row_cnt[C::RW];
  float row_tau[C::RW];
  uint32_t need_mask;
  int item;
};

// k-th largest order-preserving key (kp >= 1) among the n floats vals[0..n),
// computed by one wave: MSB radix select below the bits all entries share.
__device__ uint32_t wave_kth_key(const float* vals, int n, int kp, uint32_t* hist) {
  const int lane = __lane_id();
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
  for (int i = lane; i < n; i += 64) {
    const uint32_t k = ordered_key(vals[i]);
    lo = min(lo, k);
    hi = max(hi, k);
  }
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
  if (lo == hi) return lo;
  const int top = 31 - __clz(lo ^ hi);
  uint32_t pmask = (top == 31) ? 0u : (0xFFFFFFFFu << (top + 1));
  uint32_t prefix = hi & pmask;
  int need = kp;
  for (int bit = top; bit >= 0;) {
    const int nb = bit + 1 < 8 ? bit + 1 : 8;
    const int shift = bit + 1 - nb;
    const uint32_t dm = (1u << nb) - 1u;
#pragma unroll
    for (int b = 0; b < 4; ++b) hist[4 * lane + b] = 0u;
    for (int i = lane; i < n; i += 64) {
      const uint32_t k = ordered_key(vals[i]);
      if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & dm], 1u);
    }
    uint32_t h[4], sum = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      h[b] = hist[4 * lane + b];
      sum += h[b];
    }
    uint32_t incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t t = (uint32_t)__shfl_down((int)incl, o);
      if (lane + o < 64) incl += t;
    }
    uint32_t cum = incl - sum;
    int dig = -1, above = 0;
#pragma unroll
    for (int b = 3; b >= 0; --b) {
      if (cum < (uint32_t)need && cum + h[b] >= (uint32_t)need) {
        dig = 4 * lane + b;
        above = (int)cum;
      }
      cum += h[b];
    }
    const uint64_t who = ballot64(dig >= 0);
    const int src = __ffsll((long long)who) - 1;
    dig = __builtin_amdgcn_readlane(dig, src);
    above = __builtin_amdgcn_readlane(above, src);
    need -= above;
    prefix |= (uint32_t)dig << shift;
    pmask |= dm << shift;
    bit -= nb;
  }
  return prefix;
}

template <bool FP8> struct Opnd;
template <> struct Opnd<true> { typedef v8i T; };
template <> struct Opnd<false> { typedef v8bf T; };

template <bool FP8>
__device__ __forceinline__ typename Opnd<FP8>::T load_opnd(const uint8_t* p) {
  if constexpr (FP8) {
    v4i a = *reinterpret_cast<const v4i*>(p);
    v4i b = *reinterpret_cast<const v4i*>(p + 16);
    return v8i{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  } else {
    v4i a = *reinterpret_cast<const v4i*>(p);
    return __builtin_bit_cast(v8bf, a);
  }
}

template <bool FP8>
__device__ __forceinline__ typename Opnd<FP8>::T zero_opnd() {
  if constexpr (FP8) {
    return v8i{0, 0, 0, 0, 0, 0, 0, 0};
  } else {
    return __builtin_bit_cast(v8bf, v4i{0, 0, 0, 0});
  }
}

template <bool FP8>
__device__ __forceinline__ v16f mma(typename Opnd<FP8>::T a, typename Opnd<FP8>::T b, v16f c) {
  if constexpr (FP8) return mfma_fp8(a, b, c);
  else return mfma_bf16(a, b, c);
}

}  // namespace

template <int DT, int H, int D, bool DENSE>
__global__ void __launch_bounds__(NT, 1) prefill_kernel(PrefillParams p) {
  using C = PfCfg<DT, H, D>;
  using OT = typename Opnd<C::FP8>::T;
  __shared__ PfShared<DT, H, D> sh;
  // dynamic LDS: the list being selected (scores, then indices), or during the
  // sample phase the sampled scores of every row (RW rows x sample_m floats)
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn_lds[];
  float* lsc = reinterpret_cast<float*>(dyn_lds);
  int* lix = reinterpret_cast<int*>(dyn_lds + (size_t)p.cap * sizeof(float));
  float* smp = reinterpret_cast<float*>(dyn_lds);

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int kh = lane >> 5;      // lane half: K half of the operands, query half of the result
  const int col = lane & 31;     // MFMA row (A operand) / column (B operand, result)

  const size_t slot_elems = (size_t)C::RW * p.cap;
  float* wsc = p.ws_sc + (size_t)blockIdx.x * slot_elems;
  int* wix = p.ws_ix + (size_t)blockIdx.x * slot_elems;
  const int L = p.L;

  // A-operand row `col` of block mb holds (query slot, head) of the result row
  // with the same index: result row m has lane half (m>>2)&1 and register
  // j = 4*(m>>3) + (m&3).
  const int a_hf = (col >> 2) & 1;
  const int a_j = ((col >> 3) << 2) | (col & 3);
  const int a_slot = a_hf * C::QPH + a_j / C::HB;
  const int a_head_lo = a_j % C::HB;

  if (tid == 0) sh.need_mask = 0u;

  for (;;) {
    if (tid == 0) sh.item = atomicAdd(p.counter, 1);
    __syncthreads();
    const int item = sh.item;
    if (item >= p.n_items) break;
    const int t0 = (p.n_items - 1 - item) * C::RW;
    const int kend = min(t0 + C::RW, L);
    const int ntiles = (kend + TK - 1) / TK;

    // ---- query operands and folded head weights (registers for the whole item)
    OT qa[C::MB][C::KS];
    {
      const int t = t0 + wave * C::QPW + a_slot;
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) {
        const int head = 16 * mb + a_head_lo;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
          if (t < L) {
            const uint8_t* src = p.q + ((size_t)t * H + head) * C::ROWB + kh * (C::ROWB / 2) + ks * C::SB;
            qa[mb][ks] = load_opnd<C::FP8>(src);
          } else {
            qa[mb][ks] = zero_opnd<C::FP8>();
          }
        }
      }
    }
    float wr[C::MB][16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int t = t0 + wave * C::QPW + kh * C::QPH + j / C::HB;
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) {
        const int head = 16 * mb + j % C::HB;
        float v = 0.f;
        if (t < L) {
          v = bf16_to_f32(p.w[(size_t)t * H + head]);
          if (p.q_scale) v *= p.q_scale[(size_t)t * p.qs_row + (size_t)head * p.qs_head];
        }
        wr[mb][j] = v;
      }
    }
    const int row_base = wave * C::QPW + kh * C::QPH;   // local row of slot r is row_base + r
    float* smp_lane = smp + (size_t)row_base * p.sample_m + col;

    // ---- key tile staging.  Loads are unconditional: keys past the end read
    // the last key (such keys are always masked), so no branch merges into
    // gbuf and no early wait is forced on the prefetch.
    v4i gbuf[C::CPT];
    float gks = 1.f;
    auto gload = [&](int kt) {
#pragma unroll
      for (int c = 0; c < C::CPT; ++c) {
        const int ci = min(tid + c * NT, C::CHUNKS - 1);
        const int key = min(kt + ci / (C::ROWB / 16), L - 1);
        gbuf[c] = *reinterpret_cast<const v4i*>(p.k + (size_t)key * C::ROWB + (ci % (C::ROWB / 16)) * 16);
      }
      gks = p.k_scale ? p.k_scale[min(kt + (tid & (TK - 1)), L - 1)] : 1.f;
    };
    auto lstore = [&](int buf) {
#pragma unroll
      for (int c = 0; c < C::CPT; ++c) {
        const int ci = tid + c * NT;
        if (ci < C::CHUNKS) {
          const int kl = ci / (C::ROWB / 16);
          *reinterpret_cast<v4i*>(&sh.ktile[buf][kl * C::STRIDE + (ci % (C::ROWB / 16)) * 16]) = gbuf[c];
        }
      }
      if (tid < TK) sh.kscale[buf][tid] = gks;
    };

    // ---- scores of this lane's key column of subtile `sub` of LDS tile `buf`
    auto subtile_scores = [&](int buf, int sub, float (&score)[C::QPH]) {
      const uint8_t* bp = &sh.ktile[buf][(32 * sub + col) * C::STRIDE + kh * (C::ROWB / 2)];
      OT b[C::KS];
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) b[ks] = load_opnd<C::FP8>(bp + ks * C::SB);
      // head-weighted ReLU sum, in-lane; one 32-head block at a time so that
      // the epilogue of block mb overlaps the MFMAs of block mb+1
      float part[C::QPH][4];
#pragma unroll
      for (int r = 0; r < C::QPH; ++r)
#pragma unroll
        for (int u = 0; u < 4; ++u) part[r][u] = 0.f;
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) {
        v16f acc = v16f{};
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) acc = mma<C::FP8>(qa[mb][ks], b[ks], acc);
#pragma unroll
        for (int j = 0; j < 16; ++j)
          part[j / C::HB][j & 3] = fmaf(wr[mb][j], fmaxf(acc[j], 0.f), part[j / C::HB][j & 3]);
      }
      const float ksc = sh.kscale[buf][32 * sub + col];
#pragma unroll
      for (int r = 0; r < C::QPH; ++r) score[r] = ((part[r][0] + part[r][1]) + (part[r][2] + part[r][3])) * ksc;
    };

    // A work item runs once with a threshold estimated from a key sample and,
    // only if that estimate proved too high for some row, once more without.
    for (int attempt = 0; attempt < 2; ++attempt) {
      // The first smp_tiles iterations of the tile loop score evenly spaced
      // key tiles below t0 (valid for every row of the item) into LDS; their
      // scores give a conservative estimate tau0 of each row's k-th score.
      // The remaining iterations stream the causal prefix in key order.
      const int smp_tiles = (attempt == 0 && t0 >= 4 * p.topk) ? min(p.sample_m / TK, t0 / (8 * TK)) : 0;
      const int stile = smp_tiles >= 4 ? smp_tiles : 0;
      const int stride = stile ? (t0 / stile) / TK * TK : 0;
      const int total = stile + ntiles;
      auto tile_key = [&](int i) { return i < stile ? i * stride : (i - stile) * TK; };

      float tau0[C::QPH];   // sample threshold (inclusive), -inf without a sample
      int cnt[C::QPH];      // list length of each of this lane's rows (uniform in the lane half)
      int scnt[C::QPH];     // entries staged in LDS during the current tile
      float tau[C::QPH];    // k-th best score after the last compaction (-inf before)
#pragma unroll
      for (int r = 0; r < C::QPH; ++r) {
        tau0[r] = -__builtin_inff();
        cnt[r] = 0;
        scnt[r] = 0;
        tau[r] = -__builtin_inff();
      }

      gload(tile_key(0));
      lstore(0);
      __syncthreads();

      for (int it = 0; it < total; ++it) {
        const int kt = tile_key(it);
        const bool sampling = it < stile;
        const int buf = it & 1;
        if (it + 1 < total) gload(tile_key(it + 1));

#pragma unroll
        for (int sub = 0; sub < TK / 32; ++sub) {
          const int s0 = kt + 32 * sub;
          if (sampling || s0 < kend) {
            float sc[C::QPH];
            subtile_scores(buf, sub, sc);
            const int s = s0 + col;
            if (sampling) {
#pragma unroll
              for (int r = 0; r < C::QPH; ++r) smp_lane[r * p.sample_m + it * TK + 32 * sub] = sc[r];
            } else {
#pragma unroll
              for (int r = 0; r < C::QPH; ++r) {
                const float score = sc[r];
                const int tr = t0 + row_base + r;
                const bool valid = (s <= tr) && (tr < L);
                if constexpr (DENSE) {
                  if (attempt == 0 && tr < L && s < L) p.out_dense[(size_t)tr * L + s] = valid ? score : -__builtin_inff();
                }
                // tau: strict (later keys lose ties to the kept ones); tau0: inclusive
                const bool pass = valid && score > tau[r] && score >= tau0[r];
                const uint64_t m = ballot64(pass);
                const uint32_t mh = kh ? (uint32_t)(m >> 32) : (uint32_t)m;
                if (pass) {
                  const int pos = scnt[r] + __popc(mh & ((1u << col) - 1u));
                  sh.stage_sc[row_base + r][pos] = score;
                  sh.stage_ix[row_base + r][pos] = s;
                }
                scnt[r] += __popc(mh);
              }
            }
          }
        }

        if (!sampling) {
          // ---- move this tile's staged candidates to the rows' lists (one burst per row)
#pragma unroll
          for (int rr = 0; rr < C::QPW; ++rr) {
            const int hf = rr / C::QPH, r = rr % C::QPH;
            const int n = __builtin_amdgcn_readlane(scnt[r], hf * 32);
            const int c0 = __builtin_amdgcn_readlane(cnt[r], hf * 32);
            const int row = wave * C::QPW + rr;
            for (int e = lane; e < n; e += 64) {
              wsc[(size_t)row * p.cap + c0 + e] = sh.stage_sc[row][e];
              wix[(size_t)row * p.cap + c0 + e] = sh.stage_ix[row][e];
            }
          }
#pragma unroll
          for (int r = 0; r < C::QPH; ++r) {
            cnt[r] += scnt[r];
            scnt[r] = 0;
            // room for one more tile in every list, else ask for a compaction
            if (col == 0 && cnt[r] + TK > p.cap) {
              sh.row_cnt[row_base + r] = cnt[r];
              atomicOr(&sh.need_mask, 1u << (row_base + r));
            }
          }
        }
        if (it + 1 < total) lstore(buf ^ 1);
        __syncthreads();
        if (it == stile - 1) {
          // k' = expected sample count above the row's k-th score + 4.5 sigma:
          // the k'-th sample score is below the true k-th score except with
          // probability ~1e-5, and the end-of-item check catches that case.
          const int m = stile * TK;
#pragma unroll
          for (int rr = 0; rr < C::QPW; ++rr) {
            const int hf = rr / C::QPH, r = rr % C::QPH;
            const int t = t0 + wave * C::QPW + rr;
            const float pk = (float)p.topk / (float)(t + 1);
            const float mu = (float)m * pk;
            const int kp = (int)ceilf(mu + 4.5f * sqrtf(mu * (1.f - pk)) + 2.f);
            float v = -__builtin_inff();
            if (t < L && kp <= m / 2) {
              const uint32_t key =
                  wave_kth_key(smp + (size_t)(wave * C::QPW + rr) * p.sample_m, m, kp, sh.whist[wave]);
              v = key_to_float(key);
            }
            if (kh == hf) tau0[r] = v;
          }
          __syncthreads();
        }
        const uint32_t mask = sh.need_mask;
        if (mask) {
          for (int rl = 0; rl < C::RW; ++rl) {
            if ((mask >> rl) & 1u) {
              float* rs = wsc + (size_t)rl * p.cap;
              int* ri = wix + (size_t)rl * p.cap;
              const int n = block_select<NT>(rs, ri, sh.row_cnt[rl], p.topk, rs, ri, 0, sh.sel, lsc, lix,
                                             &sh.row_tau[rl]);
              if (tid == 0) sh.row_cnt[rl] = n;
              __syncthreads();
            }
          }
#pragma unroll
          for (int r = 0; r < C::QPH; ++r) {
            if ((mask >> (row_base + r)) & 1u) {
              cnt[r] = sh.row_cnt[row_base + r];
              tau[r] = sh.row_tau[row_base + r];
            }
          }
          __syncthreads();
          if (tid == 0) sh.need_mask = 0u;
          __syncthreads();
        }
      }

      // ---- a row is exact iff at least min(k, t+1) candidates reached its list
#pragma unroll
      for (int r = 0; r < C::QPH; ++r)
        if (col == 0) sh.row_cnt[row_base + r] = cnt[r];
      __syncthreads();
      bool short_row = false;
      for (int rl = 0; rl < C::RW; ++rl) {
        const int t = t0 + rl;
        if (t < L && sh.row_cnt[rl] < min(p.topk, t + 1)) short_row = true;
      }
      if (short_row) {          // uniform: every thread read the same counts
        __syncthreads();
        continue;               // recompute the item without the sample threshold
      }

      // ---- final selection, written to the output rows in ascending key order
      for (int rl = 0; rl < C::RW; ++rl) {
        const int t = t0 + rl;
        if (t >= L) break;
        int* dix = p.out_idx + (size_t)t * p.topk;
        float* dsc = p.out_score ? p.out_score + (size_t)t * p.topk : nullptr;
        block_select<NT>(wsc + (size_t)rl * p.cap, wix + (size_t)rl * p.cap, sh.row_cnt[rl], p.topk, dsc, dix,
                         p.topk, sh.sel, lsc, lix, nullptr);
      }
      break;
    }
  }
}

__global__ void prefill_prepare_kernel(int* counter, float* dense, long long n_dense) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i == 0) *counter = 0;
  if (dense) {
    for (long long j = i; j < n_dense; j += (long long)gridDim.x * blockDim.x) dense[j] = -__builtin_inff();
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

template <int DT, int H, int D, bool DENSE>
static hipError_t launch_variant(const PrefillParams& p, int grid, hipStream_t stream) {
  const size_t dyn = (size_t)p.cap * 8;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel<DT, H, D, DENSE>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((prefill_kernel<DT, H, D, DENSE>), dim3(grid), dim3(NT), dyn, stream, p);
  return hipGetLastError();
}

template <int DT, int H, int D>
static hipError_t launch_one(const PrefillParams& p, int grid, hipStream_t stream) {
  return p.out_dense ? launch_variant<DT, H, D, true>(p, grid, stream) : launch_variant<DT, H, D, false>(p, grid, stream);
}

template <int DT, int H, int D>
static size_t static_lds() {
  return sizeof(PfShared<DT, H, D>);
}

int prefill_rows_per_item(int H) { return WAVES * 2 * (H < 16 ? 16 / H : 1); }

bool prefill_supported(int dt, int H, int D) {
  const bool fp8 = dt == DSA_FP8_E4M3;
  if (!(H == 8 || H == 16 || H == 32 || H == 64)) return false;
  if (D != 64 && D != 128) return false;
  if (!fp8 && H == 64 && D == 128) return false;   // register budget
  return true;
}

int prefill_tile_keys() { return TK; }

// Keys per row sampled for the threshold estimate: the sampled scores of all
// rows of a work item live in the dynamic LDS area (2 * cap words), at most
// 1024 per row, whole tiles only; fewer than 4 tiles disables the sample.
int prefill_sample_keys(int H, int cap) {
  const int rw = prefill_rows_per_item(H);
  int m = (2 * cap / rw) / TK * TK;
  if (m > 1024) m = 1024;
  return m >= 4 * TK ? m : 0;
}

// Candidate list capacity per row: 4*topk when the LDS allows (the select
// stages one list in LDS next to the kernel's static shared memory), never
// less than topk plus one tile.  Returns 0 if no capacity fits.
int prefill_list_capacity(int dt, int H, int D, int topk) {
  size_t st = 0;
#define DSA_PF_LDS(DT_, H_, D_) \
  if (dt == DT_ && H == H_ && D == D_) st = static_lds<DT_, H_, D_>();
  DSA_PF_LDS(DSA_FP8_E4M3, 64, 128)
  DSA_PF_LDS(DSA_FP8_E4M3, 64, 64)
  DSA_PF_LDS(DSA_FP8_E4M3, 32, 128)
  DSA_PF_LDS(DSA_FP8_E4M3, 32, 64)
  DSA_PF_LDS(DSA_FP8_E4M3, 16, 128)
  DSA_PF_LDS(DSA_FP8_E4M3, 16, 64)
  DSA_PF_LDS(DSA_FP8_E4M3, 8, 128)
  DSA_PF_LDS(DSA_FP8_E4M3, 8, 64)
  DSA_PF_LDS(DSA_BF16, 64, 64)
  DSA_PF_LDS(DSA_BF16, 32, 128)
  DSA_PF_LDS(DSA_BF16, 32, 64)
  DSA_PF_LDS(DSA_BF16, 16, 128)
  DSA_PF_LDS(DSA_BF16, 16, 64)
  DSA_PF_LDS(DSA_BF16, 8, 128)
  DSA_PF_LDS(DSA_BF16, 8, 64)
#undef DSA_PF_LDS
  if (st == 0) return 0;
  const size_t lds_limit = 160 * 1024;
  if (st + 8 * (size_t)(topk + TK) > lds_limit) return 0;
  size_t cap = 4 * (size_t)topk;
  if (cap < (size_t)topk + 16 * TK) cap = (size_t)topk + 16 * TK;
  const size_t max_cap = (lds_limit - st) / 8 / 64 * 64;
  if (cap > max_cap) cap = max_cap;
  cap = cap / 64 * 64;
  if (cap < (size_t)topk + TK) return 0;
  return (int)cap;
}

hipError_t prefill_launch(const PrefillParams& p, int dt, int H, int D, int grid, hipStream_t stream) {
  const long long n_dense = p.out_dense ? (long long)p.L * p.L : 0;
  const int pg = n_dense ? 1024 : 1;
  hipLaunchKernelGGL(prefill_prepare_kernel, dim3(pg), dim3(256), 0, stream, p.counter, p.out_dense, n_dense);
#define DSA_PF_CASE(DT_, H_, D_) \
  if (dt == DT_ && H == H_ && D == D_) return launch_one<DT_, H_, D_>(p, grid, stream);
  DSA_PF_CASE(DSA_FP8_E4M3, 64, 128)
  DSA_PF_CASE(DSA_FP8_E4M3, 64, 64)
  DSA_PF_CASE(DSA_FP8_E4M3, 32, 128)
  DSA_PF_CASE(DSA_FP8_E4M3, 32, 64)
  DSA_PF_CASE(DSA_FP8_E4M3, 16, 128)
  DSA_PF_CASE(DSA_FP8_E4M3, 16, 64)
  DSA_PF_CASE(DSA_FP8_E4M3, 8, 128)
  DSA_PF_CASE(DSA_FP8_E4M3, 8, 64)
  DSA_PF_CASE(DSA_BF16, 64, 64)
  DSA_PF_CASE(DSA_BF16, 32, 128)
  DSA_PF_CASE(DSA_BF16, 32, 64)
  DSA_PF_CASE(DSA_BF16, 16, 128)
  DSA_PF_CASE(DSA_BF16, 16, 64)
  DSA_PF_CASE(DSA_BF16, 8, 128)
  DSA_PF_CASE(DSA_BF16, 8, 64)
#undef DSA_PF_CASE
  return hipErrorInvalidValue;
}

}  // namespace dsa
