// Fused prefill lightning indexer + streaming top-k for gfx950.
//
// What is computed (IndexCache deep-dive report, abstract and section 1.1:
// a multi-head ReLU-gated dot product, run in FP8, that scores every earlier
// token and keeps the k best):
//   score(t, s) = k_scale[s] * sum_h w[t,h] * q_scale[t,h] * ReLU(q[t,h] . k[s]),  s <= t
// and, per query row t, the min(k, t+1) best keys under "score descending,
// key index ascending", written in ascending key order and padded with -1.
//
// Design (one work item = RW consecutive query rows, 8 waves; 4 waves, one
// per SIMD, for the configurations whose registers do not fit two waves per
// SIMD: H = 128, and bf16 at H = 64 with D = 128):
// * Score contraction on MFMA.  Index heads sit on the MFMA row dimension and
//   keys on the column dimension.  With the 32x32 accumulator layout a lane
//   owns one key column and 16 rows of each 32-row block.
//   H >= 32: a wave serves one query; block i holds heads 32i..32i+31, so the
//   two lane halves hold different heads of the same query.  After the
//   in-lane head sums the halves trade one partial sum per pair of 32-key
//   subtiles, which leaves every lane with the full score of a distinct key.
//   H <= 16: the rows of the single block belong to one query per lane half
//   (two queries of 8 heads for H == 8): no cross-lane step at all.
//   fp8 path: v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3 x e4m3, unit block
//   scales); bf16 path: v_mfma_f32_32x32x16_bf16.  Products are exact, the
//   accumulation is fp32.
// * Keys are staged through LDS in tiles of 256 keys (128 when a key row is
//   wider than 128 bytes or H <= 16), double buffered, with direct
//   global-to-LDS loads into swizzled rows; every wave reuses each tile for
//   its own queries.  Query operands and the folded head
//   weights w*q_scale stay in registers for the whole work item.  Inside a
//   tile the MFMAs of one head block overlap the VALU epilogue of the
//   previous one (two accumulators, explicit issue groups).
// * Epilogue per (query, key): sum_h w_eff * max(x, 0), times k_scale, causal
//   mask.  The L x L score matrix is never stored (the optional dense output
//   exists for small debugging runs only).
// * Streaming top-k: each row keeps a threshold (the larger of the current
//   k-th best score tau and a sample estimate tau0) and appends keys strictly
//   above it, in ascending key order, to a candidate list in the
//   per-workgroup workspace.  Keys arrive in ascending index order, so a
//   later key that ties the k-th score always loses the tie and "strictly
//   greater" is exact for tau.  tau0 comes from scoring a strided sample of
//   keys first; a row whose list ends shorter than min(k, t+1) may have lost
//   keys to it, and its item is recomputed without the sample.  When a list
//   could overflow during the next tile, the wave that owns it compacts it to
//   exactly k entries (a wave-level radix select), which also raises tau.  At
//   the end of the work item the same routine selects the final k of each
//   row and writes them out in order.
// * Persistent grid: one workgroup per CU pulls work items from an atomic
//   counter, longest (highest t) first, which balances the causal triangle.
//   A work item whose rows all have t + 1 <= k keeps every key; when the
//   caller wants no scores it is written out without being scored.
// * Query rows need not start at position 0: a chunk (query offset q0) or a
//   ragged batch (a device table of items, each naming its sequence's key
//   rows, key count, q row offset and first position) reads its rows at
//   t + offset and its keys from its own sequence; positions, tiles and the
//   causal mask stay absolute.
#include "device_common.hpp"
#include "wave_select.hpp"
#include "kernels.hpp"

namespace dsa {

namespace {

template <int DT, int H, int D>
struct PfCfg {
  static constexpr bool FP8 = (DT == DSA_FP8_E4M3);
  // one wave per SIMD where a wave's registers exceed half the SIMD's file:
  // the query operands, head weights and accumulators of 128 heads, or the
  // eight 16-deep bf16 K steps (operands and B ring) of a 128-wide row
  static constexpr bool WIDE = H == 128 || (!FP8 && H == 64 && D == 128);
  static constexpr int NT = WIDE ? 256 : 512;       // threads per workgroup
  static constexpr int WAVES = NT / 64;
  // H >= 32: one query per wave; each 32-row MFMA block holds 32 of its heads,
  // so the two lane halves hold different heads of the same query and one
  // cross-half add finishes the head sum.  H <= 16: each lane half holds its
  // own queries (16/H of them) and the head sum stays inside a lane.
  static constexpr bool SPLIT = H >= 32;
  static constexpr int HB = H < 16 ? H : 16;        // heads of one query in one lane-block (H <= 16)
  static constexpr int QPH = SPLIT ? 1 : 16 / HB;   // query slots per lane
  static constexpr int QPW = SPLIT ? 1 : 2 * QPH;   // queries per wave
  static constexpr int MB = SPLIT ? H / 32 : 1;     // 32-row MFMA blocks per wave
  static constexpr int ESZ = FP8 ? 1 : 2;           // bytes per element
  static constexpr int KM = FP8 ? 64 : 16;          // K of one MFMA
  static constexpr int KS = D / KM;                 // MFMAs along D
  static constexpr int SB = FP8 ? 32 : 16;          // bytes per lane per MFMA operand
  static constexpr int ROWB = D * ESZ;              // bytes of one key / one query head
  // keys per LDS tile: 256 for one query per wave and key rows of at most
  // 128 bytes (halves the per-tile barriers), else 128 (LDS budget)
  static constexpr int TK = (ROWB <= 128 && SPLIT) ? 256 : 128;
  static constexpr int RW = WAVES * QPW;            // query rows per work item
  // LDS key tile: rows of ROWB bytes, unpadded; the 16-byte chunks of row r
  // sit at chunk position c ^ swz(r), swz(r) = (r / RPB) & (CPR - 1), so the
  // 16 lanes that read one chunk of 16 consecutive rows in a ds_read_b128
  // cycle hit 16 different 16-byte bank groups of the 64-bank LDS.
  static constexpr int CPR = ROWB / 16;             // 16-byte chunks per key row
  static constexpr int RPB = 256 / ROWB;            // key rows per 256-byte bank sweep
  static constexpr int NLD = TK * ROWB / 1024;      // 1 KB direct-to-LDS loads per tile
  static_assert(ROWB <= 256 && NLD % WAVES == 0, "tile layout");
  static_assert(H == 8 || H == 16 || H == 32 || H == 64 || H == 128, "unsupported head count");
  static_assert(D % KM == 0 && ROWB / 2 == KS * SB, "unsupported head dim");
  static_assert(RW <= 32, "row mask is 32 bits");
  // query slot of accumulator register j (result row 8(j/4) + 4*half + j%4)
  static __device__ __forceinline__ int slot_of(int j) { return SPLIT ? 0 : j / HB; }
};

// The key tiles and the candidate stage come last, so that together with the
// dynamic sample area that follows the static block they form one span of
// LDS that the end-of-item selection reuses as per-wave scratch.
template <int DT, int H, int D>
struct PfShared {
  using C = PfCfg<DT, H, D>;
  __attribute__((aligned(16))) float kscale[2][C::TK];
  uint32_t whist[C::WAVES][256];           // per-wave radix histogram (selection, sample quantile)
  __attribute__((aligned(16))) float weff[C::RW * H];   // folded head weights w*q_scale of the item's rows
  int row_cnt[C::RW];
  int item;
  __attribute__((aligned(1024))) uint8_t ktile[2][C::TK * C::ROWB];   // double-buffered key tile (swizzled)
  __attribute__((aligned(16))) float stage_sc[C::RW][C::TK];          // this tile's accepted candidates, per row
  int stage_ix[C::RW][C::TK];
};

// Dynamic LDS of a launch: the rest of the CU's 160 KB after the static
// block, less 1 KB of slack (at least the threshold sample's RW x sample_m
// floats, which are 32 KB at most).  The end-of-item selection uses all of
// it as scratch for the rows' candidate scores.
template <int DT, int H, int D>
constexpr size_t pf_dyn_bytes() {
  return sizeof(PfShared<DT, H, D>) + 1024 >= 160 * 1024 ? 0 : (160 * 1024 - sizeof(PfShared<DT, H, D>) - 1024) / 1024 * 1024;
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
__global__ void __launch_bounds__((PfCfg<DT, H, D>::NT), 1) prefill_kernel(PrefillParams p) {
  using C = PfCfg<DT, H, D>;
  constexpr int NT = C::NT;
  constexpr int WAVES = C::WAVES;
  using OT = typename Opnd<C::FP8>::T;
  __shared__ PfShared<DT, H, D> sh;
  // dynamic LDS: the sampled scores of every row (RW rows x sample_m floats)
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn_lds[];
  float* smp = reinterpret_cast<float*>(dyn_lds);

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int kh = lane >> 5;      // lane half: K half of the operands, query half of the result
  const int col = lane & 31;     // MFMA row (A operand) / column (B operand, result)

  const size_t slot_elems = (size_t)C::RW * p.cap;
  float* wsc = p.ws_sc + (size_t)blockIdx.x * slot_elems;
  int* wix = p.ws_ix + (size_t)blockIdx.x * slot_elems;

  // A-operand row `col` of block mb holds the (query slot, head) of the result
  // row with the same index: result row m has lane half (m>>2)&1 and register
  // j = 4*(m>>3) + (m&3).
  const int a_hf = (col >> 2) & 1;
  const int a_j = ((col >> 3) << 2) | (col & 3);
  const int a_slot = C::SPLIT ? 0 : a_hf * C::QPH + a_j / C::HB;
  const int a_head = C::SPLIT ? col : a_j % C::HB;   // head within block mb (block stride 32 or 16)
  constexpr int HSTRIDE = C::SPLIT ? 32 : 16;

  for (;;) {
    if (tid == 0) sh.item = atomicAdd(p.counter, 1);
    __syncthreads();
    const int item = sh.item;
    // the item's sequence: key count L, its keys, and the q/w/output row of
    // query position t (t + qoff)
    int L, t0, qoff;
    const uint8_t* kp;
    const float* ksp;
    if (p.items) {
      if (item >= *p.n_items_dev) break;
      const int4 it = p.items[item];
      qoff = it.x;
      kp = p.k + (size_t)it.y * C::ROWB;
      ksp = p.k_scale ? p.k_scale + it.y : nullptr;
      L = it.z;
      t0 = it.w;
    } else {
      if (item >= p.n_items) break;
      qoff = -p.q0;
      kp = p.k;
      ksp = p.k_scale;
      L = p.L;
      t0 = p.q0 + (p.n_items - 1 - item) * C::RW;
    }
    // Every row of the item has at most topk keys: its selection is all of
    // them, 0 .. t in order.  Without requested scores nothing needs scoring.
    if (!DENSE && p.out_score == nullptr && t0 + C::RW <= p.topk) {
      for (int rl = wave; rl < C::RW; rl += WAVES) {
        const int t = t0 + rl;
        if (t >= L) break;
        int* dix = p.out_idx + (size_t)(t + qoff) * p.topk;
        for (int j = lane; j < p.topk; j += 64) __builtin_nontemporal_store(j <= t ? j : -1, dix + j);
      }
      __syncthreads();   // every thread has read sh.item before the next one is taken
      continue;
    }
    const int kend = min(t0 + C::RW, L);
    const int ntiles = (kend + C::TK - 1) / C::TK;

    // ---- query operands and folded head weights (registers for the whole item)
    OT qa[C::MB][C::KS];
    {
      const int t = t0 + wave * C::QPW + a_slot;
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) {
        const int head = HSTRIDE * mb + a_head;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
          if (t < L && head < p.hr) {
            const uint8_t* src = p.q + ((size_t)(t + qoff) * p.hr + head) * C::ROWB + kh * (C::ROWB / 2) + ks * C::SB;
            qa[mb][ks] = load_opnd<C::FP8>(src);
          } else {
            qa[mb][ks] = zero_opnd<C::FP8>();
          }
        }
      }
    }
    // folded head weights w*q_scale of the item's rows, staged once in LDS
    // with coalesced loads, then 16 per block into registers
    for (int i = tid; i < C::RW * H; i += NT) {
      const int t = t0 + i / H, head = i % H;
      float v = 0.f;
      if (t < L && head < p.hr) {
        v = bf16_to_f32(p.w[(size_t)(t + qoff) * p.hr + head]);
        if (p.q_scale) v *= p.q_scale[(size_t)(t + qoff) * p.qs_row + (size_t)head * p.qs_head];
      }
      sh.weff[i] = v;
    }
    __syncthreads();
    float wr[C::MB][16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int slot = C::SPLIT ? 0 : kh * C::QPH + j / C::HB;
      const int row = wave * C::QPW + slot;
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) {
        const int head = C::SPLIT ? 32 * mb + 8 * (j >> 2) + 4 * kh + (j & 3) : j % C::HB;
        wr[mb][j] = sh.weff[row * H + head];
      }
    }
    const int row_base = wave * C::QPW + (C::SPLIT ? 0 : kh * C::QPH);   // local row of slot r is row_base + r
    float* smp_lane = smp + (size_t)row_base * p.sample_m + col;
    float* smp_row = smp + (size_t)wave * p.sample_m;   // H >= 32: the wave's single row

    // ---- key tile staging: direct global -> LDS loads (no registers, no
    // copy), 1 KB per wave instruction: lane i of load g fills chunk position
    // 64g + i of the tile.  Keys past the end read the last key (always
    // masked), so every load is unconditional.  Completion is awaited (vmcnt)
    // right before the barrier that publishes the tile.
    auto issue_tile = [&](int kt, uint8_t* tdst, float* kdst) {
#pragma unroll
      for (int i = 0; i < C::NLD / WAVES; ++i) {
        const int g = wave + WAVES * i;
        const int pos = 64 * g + lane;
        const int r = pos / C::CPR;
        const int c = (pos % C::CPR) ^ ((r / C::RPB) & (C::CPR - 1));
        const uint8_t* src = kp + (size_t)min(kt + r, L - 1) * C::ROWB + c * 16;
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                         (__attribute__((address_space(3))) void*)(tdst + 1024 * g), 16, 0, 0);
      }
      if (wave < C::TK / 64) {
        // H >= 32 reads k_scale lane-major: key 64*pair + lane at lane*(TK/64) + pair
        const int pos = 64 * wave + lane;
        const int kk = C::SPLIT ? 64 * (pos % (C::TK / 64)) + pos / (C::TK / 64) : pos;
        if (ksp) {
          __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(ksp + min(kt + kk, L - 1)),
                                           (__attribute__((address_space(3))) void*)(kdst + 64 * wave), 4, 0, 0);
        } else {
          kdst[pos] = 1.f;
        }
      }
    };
    // this lane's B-operand chunk offsets within a key row (the swizzle only
    // depends on the row modulo 32, i.e. on the lane)
    const int bswz = (col / C::RPB) & (C::CPR - 1);
    int boff[C::KS][C::FP8 ? 2 : 1];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
      for (int h = 0; h < (C::FP8 ? 2 : 1); ++h)
        boff[ks][h] = ((((kh * (C::ROWB / 2) + ks * C::SB) >> 4) + h) ^ bswz) * 16;

    // ---- scores of all 32-key subtiles of LDS tile `buf`.  One straight-line
    // block: two accumulator sets alternate between subtiles so the MFMAs of
    // subtile i+1 run while the VALU epilogue of subtile i executes, and the
    // B operand of the next subtile is fetched from LDS during the current one.
    //   H <= 16: on_score(sub, score[QPH]) per subtile; lane (half, col) holds
    //            key 32*sub + col of its half's query slots.
    //   H >= 32: on_score(pair, score) per subtile pair; the halves trade
    //            partial head sums so that lane l holds the full score of key
    //            64*pair + l (half 0 finishes the even subtile, half 1 the odd).
    auto tile_scores = [&](const uint8_t* tile, const float* ksc_t, auto&& on_score) {
      const uint8_t* bp = tile + col * C::ROWB;
      auto load_b = [&](int sub, int ks) -> OT {
        const uint8_t* rp = bp + 32 * sub * C::ROWB;
        if constexpr (C::FP8) {
          const v4i lo = *reinterpret_cast<const v4i*>(rp + boff[ks][0]);
          const v4i hi = *reinterpret_cast<const v4i*>(rp + boff[ks][C::FP8 ? 1 : 0]);
          return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        } else {
          return __builtin_bit_cast(v8bf, *reinterpret_cast<const v4i*>(rp + boff[ks][0]));
        }
      };
      constexpr int NSUB = C::TK / 32;
      // B operands, three subtiles deep: the buffer refilled for subtile
      // i+1 was last read by the MFMAs of subtile i-2, long complete, so the
      // refill never waits on an MFMA still reading its registers
      OT b[3][C::KS];
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) b[0][ks] = load_b(0, ks);
      v16f acc[2][C::MB];
      float part[C::QPH][4];
      float even_half = 0.f;   // H >= 32: this half's partial sum of the even subtile
      // Each finished score is handed to on_score one subtile later, so its
      // dependent filter chain issues between the next subtile's MFMAs.
      float pend_sc[C::QPH];
      int pend_id = -1;
      auto flush_pending = [&]() {
        if (pend_id >= 0) {
          if constexpr (C::SPLIT) on_score(pend_id, pend_sc[0]);
          else on_score(pend_id, pend_sc);
        }
      };
      // H >= 32: k_scale of key 64*pair + lane for every pair of the tile
      // (stored lane-major, one vector read)
      float ksc_v[C::TK / 64];
      if constexpr (C::SPLIT) {
        const float* kp = ksc_t + lane * (C::TK / 64);
        if constexpr (C::TK == 256) {
          const float4 v = *reinterpret_cast<const float4*>(kp);
          ksc_v[0] = v.x; ksc_v[1] = v.y; ksc_v[2] = v.z; ksc_v[3] = v.w;
        } else {
          const float2 v = *reinterpret_cast<const float2*>(kp);
          ksc_v[0] = v.x; ksc_v[1] = v.y;
        }
      }
      // epilogue of subtile `sub` (its accumulators for every head block)
      auto epilogue = [&](int sub) {
        const v16f* a = acc[sub & 1];
#pragma unroll
        for (int r = 0; r < C::QPH; ++r)
#pragma unroll
          for (int u = 0; u < 4; ++u) part[r][u] = 0.f;
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
          for (int j = 0; j < 16; ++j)
            part[C::slot_of(j)][j & 3] = fmaf(wr[mb][j], fmaxf(a[mb][j], 0.f), part[C::slot_of(j)][j & 3]);
        if constexpr (C::SPLIT) {
          const float h = (part[0][0] + part[0][1]) + (part[0][2] + part[0][3]);
          if ((sub & 1) == 0) {
            even_half = h;
          } else {
            // v_permlane32_swap(X = even partials, Y = odd partials) returns
            // (X[l], X[l+32]) to lanes l < 32 and (Y[l-32], Y[l]) to lanes
            // l >= 32: the two partials of key 64*pair + l, half 0 first
            const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(even_half), __float_as_uint(h),
                                                              false, false);
            const float full = __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
            pend_sc[0] = full * ksc_v[sub >> 1];
            pend_id = sub >> 1;
          }
        } else {
          const float ksc = ksc_t[32 * sub + col];
#pragma unroll
          for (int r = 0; r < C::QPH; ++r)
            pend_sc[r] = ((part[r][0] + part[r][1]) + (part[r][2] + part[r][3])) * ksc;
          pend_id = sub;
        }
      };
      // MFMAs of one subtile are issued K-step-major across the head blocks,
      // so an MFMA never waits on the one issued just before it; each is
      // followed by its share of the previous subtile's epilogue, which only
      // reads the other accumulator set.  The barrier keeps subtiles apart
      // (hoisting later MFMAs would run out of registers).
      constexpr int NMF = C::MB * C::KS;
      constexpr int VPER = (32 * C::MB + 24 + NMF - 1) / NMF;
      constexpr int NDS = C::KS * (C::FP8 ? 2 : 1);   // ds_read_b128 per subtile B operand
#pragma unroll
      for (int sub = 0; sub < NSUB; ++sub) {
        if (sub + 1 < NSUB) {
#pragma unroll
          for (int ks = 0; ks < C::KS; ++ks)
            b[(sub + 1) % 3][ks] = load_b(sub + 1, ks);
        }
        v16f c[C::MB];
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb) c[mb] = v16f{};
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
          for (int mb = 0; mb < C::MB; ++mb) c[mb] = mma<C::FP8>(qa[mb][ks], b[sub % 3][ks], c[mb]);
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb) acc[sub & 1][mb] = c[mb];
        if (sub > 0) {
          flush_pending();
          pend_id = -1;
          epilogue(sub - 1);
        }
        // next subtile's B reads first, then MFMAs each followed by a share
        // of the epilogue
        if (sub + 1 < NSUB) __builtin_amdgcn_sched_group_barrier(0x100, NDS, 0);
#pragma unroll
        for (int i = 0; i < NMF; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, VPER, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      flush_pending();
      pend_id = -1;
      epilogue(NSUB - 1);
      flush_pending();
    };

    // A work item runs once with a threshold estimated from a key sample and,
    // only if that estimate proved too high for some row, once more without.
    for (int attempt = 0; attempt < 2; ++attempt) {
      // The first smp_tiles iterations of the tile loop score evenly spaced
      // key tiles below t0 (valid for every row of the item) into LDS; their
      // scores give a conservative estimate tau0 of each row's k-th score.
      // The remaining iterations stream the causal prefix in key order.
      // (from t0 >= 3k: there a sample of at least 2 tiles already gives a
      // threshold that keeps the lists, and the end-of-item selection, short).
      // The sample grows with the prefix: one tile per 64 tiles of keys, at
      // least two, at most 1/8 of the keys and at most sample_m keys.  A
      // short row gains less from a tighter threshold than extra sample
      // tiles cost it.
      const int smp_tiles = (attempt == 0 && t0 >= 3 * p.topk)
                                ? min(min(p.sample_m / C::TK, t0 / (8 * C::TK)), max(2, t0 / (64 * C::TK)))
                                : 0;
      const int stile = smp_tiles >= 2 ? smp_tiles : 0;
      const int stride = stile ? (t0 / stile) / C::TK * C::TK : 0;
      const int total = stile + ntiles;
      auto tile_key = [&](int i) { return i < stile ? i * stride : (i - stile) * C::TK; };

      float tau0[C::QPH];   // sample threshold, -inf without a sample
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

      issue_tile(tile_key(0), sh.ktile[0], sh.kscale[0]);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();

      for (int it = 0; it < total; ++it) {
        const int kt = tile_key(it);
        const bool sampling = it < stile;
        const int buf = it & 1;
        // The two tile buffers are distinct; saying so (restrict) lets the
        // compiler read the current tile without first waiting for the load
        // of the next one into the other buffer.
        auto tile_body = [&](const uint8_t* __restrict__ tile, const float* __restrict__ ksc_t,
                             uint8_t* __restrict__ ntile, float* __restrict__ nksc) {
        if (it + 1 < total) issue_tile(tile_key(it + 1), ntile, nksc);

        // The two branches run the same MFMA sequence; the distinct markers
        // keep the compiler from hoisting it into the common predecessor,
        // where its results would stay live across the branch.
        // rows past the end of the sequence accept nothing
        float thr[C::QPH];
#pragma unroll
        for (int r = 0; r < C::QPH; ++r)
          thr[r] = (t0 + row_base + r < L) ? fmaxf(tau[r], tau0[r]) : __builtin_inff();
        if (sampling) {
          asm volatile("; sample tile" ::: "memory");
          if constexpr (C::SPLIT) {
            tile_scores(tile, ksc_t, [&](int pair, float sc) { smp_row[it * C::TK + 64 * pair + lane] = sc; });
          } else {
            tile_scores(tile, ksc_t, [&](int sub, const float (&sc)[C::QPH]) {
#pragma unroll
              for (int r = 0; r < C::QPH; ++r) smp_lane[r * p.sample_m + it * C::TK + 32 * sub] = sc[r];
            });
          }
        } else {
          asm volatile("; stream tile" ::: "memory");
          // Branch-free staging: passing lanes take the next free slots of the
          // row's stage in key order, the others fill the slots after them
          // (overwritten by the next group), so every group of keys writes
          // consecutive words.  Filter: strictly above max(tau, tau0).
          if constexpr (C::SPLIT) {
            const int tr = t0 + wave;
            tile_scores(tile, ksc_t, [&](int pair, float score) {
              const int s = kt + 64 * pair + lane;
              if constexpr (DENSE) {
                if (attempt == 0 && tr < L && s < L) p.out_dense[(size_t)(tr + qoff) * L + s] = s <= tr ? score : -__builtin_inff();
              }
              const bool pass = (s <= tr) && (score > thr[0]);
              const uint64_t m = ballot64(pass);
              const int np = __popcll(m);
              const int before = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
              const int pos = scnt[0] + (pass ? before : np + lane - before);
              sh.stage_sc[wave][pos] = score;
              sh.stage_ix[wave][pos] = s;
              scnt[0] += np;
            });
          } else {
            tile_scores(tile, ksc_t, [&](int sub, const float (&sc)[C::QPH]) {
              const int s = kt + 32 * sub + col;
              const uint32_t lt = (1u << col) - 1u;
#pragma unroll
              for (int r = 0; r < C::QPH; ++r) {
                const float score = sc[r];
                const int tr = t0 + row_base + r;
                if constexpr (DENSE) {
                  if (attempt == 0 && tr < L && s < L) p.out_dense[(size_t)(tr + qoff) * L + s] = s <= tr ? score : -__builtin_inff();
                }
                const bool pass = (s <= tr) && (score > thr[r]);
                const uint64_t m = ballot64(pass);
                const uint32_t mh = kh ? (uint32_t)(m >> 32) : (uint32_t)m;
                const int np = __popc(mh);
                const int before = __popc(mh & lt);
                const int pos = scnt[r] + (pass ? before : np + col - before);
                sh.stage_sc[row_base + r][pos] = score;
                sh.stage_ix[row_base + r][pos] = s;
                scnt[r] += np;
              }
            });
          }
        }
        };
        tile_body(sh.ktile[buf], sh.kscale[buf], sh.ktile[buf ^ 1], sh.kscale[buf ^ 1]);

        if (!sampling) {
          // ---- move this tile's staged candidates to the rows' lists (one
          // burst per row); a list without room for one more tile is
          // compacted to its k best right away by the wave that owns it
          wave_lds_sync();   // stage entries were written by other lanes
#pragma unroll
          for (int rr = 0; rr < C::QPW; ++rr) {
            const int hf = C::SPLIT ? 0 : rr / C::QPH, r = C::SPLIT ? 0 : rr % C::QPH;
            const int n = __builtin_amdgcn_readlane(scnt[r], hf * 32);
            const int c0 = __builtin_amdgcn_readlane(cnt[r], hf * 32);
            const int row = wave * C::QPW + rr;
            float* rs = wsc + (size_t)row * p.cap;
            int* ri = wix + (size_t)row * p.cap;
            for (int e = lane; e < n; e += 64) {
              rs[c0 + e] = sh.stage_sc[row][e];
              ri[c0 + e] = sh.stage_ix[row][e];
            }
            int c = c0 + n;
            if (c + C::TK > p.cap) {
              __threadfence_block();
              float tnew;
              c = wave_select(rs, ri, c, p.topk, rs, ri, 0, sh.whist[wave], &tnew);
              if (C::SPLIT || kh == hf) tau[r] = tnew;
            }
            if (C::SPLIT || kh == hf) cnt[r] = c;
          }
#pragma unroll
          for (int r = 0; r < C::QPH; ++r) scnt[r] = 0;
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's part of the next tile has landed
        __syncthreads();
        if (it == stile - 1) {
          // k' = expected sample count above the row's k-th score + 4.5 sigma:
          // the k'-th sample score is below the true k-th score except with
          // probability ~1e-5.  Any threshold is safe: a row whose list ends
          // with at least min(k, t+1) keys strictly above it holds every key
          // of its top k, and the end-of-item check redoes any other row.
          const int m = stile * C::TK;
#pragma unroll
          for (int rr = 0; rr < C::QPW; ++rr) {
            const int hf = C::SPLIT ? 0 : rr / C::QPH, r = C::SPLIT ? 0 : rr % C::QPH;
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
            if (C::SPLIT || kh == hf) tau0[r] = v;
          }
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
      // Only a sample threshold can make a row short with finite scores: the
      // item is then recomputed without it.  Without a sample (always so on
      // the second attempt) a short row has keys whose score is NaN or -inf,
      // which never pass the filter; the final selection writes what the
      // row holds and pads the rest.
      if (short_row && stile > 0) {   // uniform: every thread read the same counts
        __syncthreads();
        continue;
      }

      // ---- final selection: each wave writes its own rows, in ascending key
      // order.  The key tiles, the stage and (when it directly follows the
      // static block) the dynamic area (the sample and the rest of the LDS)
      // are free now: each wave gets an equal, 16-byte aligned share as
      // scratch for its row's scores.
      uint8_t* scr = &sh.ktile[0][0];
      const uint8_t* scr_static_end = reinterpret_cast<const uint8_t*>(&sh.stage_ix[0][0]) + sizeof(sh.stage_ix);
      size_t scr_bytes = (size_t)(scr_static_end - scr);
      // the dynamic area follows the static block (whose size is padded to
      // its 1 KB alignment): the span up to its end is this workgroup's LDS
      const uint8_t* dyn_begin = reinterpret_cast<const uint8_t*>(dyn_lds);
      const uint8_t* sh_end = reinterpret_cast<const uint8_t*>(&sh) + sizeof(sh);
      if (dyn_begin >= scr_static_end && dyn_begin <= sh_end + 16)
        scr_bytes = (size_t)(dyn_begin + pf_dyn_bytes<DT, H, D>() - scr);
      // A row whose list leaves room in the share for a 4-copy digit
      // histogram gets one at the end of the share; a longer list keeps the
      // whole share for its scores and counts into the wave's 1-copy one.
      constexpr int HCOPIES = 4;
      const int share = (int)(scr_bytes / WAVES / 16) * 4;   // floats per wave, a multiple of 4
      const int lcap_w = share - 256 * HCOPIES;
      float* lbuf = reinterpret_cast<float*>(scr) + (size_t)wave * share;
      uint32_t* fhist = reinterpret_cast<uint32_t*>(lbuf + (lcap_w > 0 ? lcap_w : 0));
#pragma unroll 1
      for (int rr = 0; rr < C::QPW; ++rr) {
        const int row = wave * C::QPW + rr;
        const int t = t0 + row;
        if (t >= L) continue;
        int* dix = p.out_idx + (size_t)(t + qoff) * p.topk;
        float* dsc = p.out_score ? p.out_score + (size_t)(t + qoff) * p.topk : nullptr;
        const int n = sh.row_cnt[row];
        if (n <= lcap_w)
          wave_select<HCOPIES, true>(wsc + (size_t)row * p.cap, wix + (size_t)row * p.cap, n, p.topk, dsc, dix,
                                     p.topk, fhist, nullptr, lbuf, lcap_w);
        else
          wave_select<1, true>(wsc + (size_t)row * p.cap, wix + (size_t)row * p.cap, n, p.topk, dsc, dix, p.topk,
                               sh.whist[wave], nullptr, lbuf, share);
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

// Ragged-batch item table (one workgroup of 1024 threads).
__global__ void __launch_bounds__(1024) prefill_varlen_prepare_kernel(const int32_t* cu_q, const int32_t* cu_k,
                                                                      int nseq, int total_q, int total_k, int rw,
                                                                      int4* items, int cap_items, int* n_items,
                                                                      int* counter) {
  __shared__ int key[1024], idx[1024], scan[1024];
  __shared__ int base;
  const int tid = threadIdx.x;
  if (tid == 0) {
    *counter = 0;
    base = 0;
  }
  // query count, key count and items of sequence i (0 when its bounds are invalid)
  auto seq = [&](int i, int& lq, int& lk) {
    const int a = cu_q[i], b = cu_q[i + 1], c = cu_k[i], d = cu_k[i + 1];
    const bool ok = 0 <= a && a <= b && b <= total_q && 0 <= c && c <= d && d <= total_k && b - a <= d - c;
    lq = ok ? b - a : 0;
    lk = ok ? d - c : 0;
    return (lq + rw - 1) / rw;
  };
  auto block_scan = [&](int v) {   // inclusive prefix sum over the workgroup
    scan[tid] = v;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {
      const int x = tid >= o ? scan[tid - o] : 0;
      __syncthreads();
      scan[tid] += x;
      __syncthreads();
    }
    return scan[tid];
  };
  auto emit = [&](int i, int off) {   // items of sequence i, its longest first
    int lq, lk;
    const int nit = seq(i, lq, lk);
    const int q0 = lk - lq;
    for (int m = 0; m < nit && off + m < cap_items; ++m)
      items[off + m] = make_int4(cu_q[i] - q0, cu_k[i], lk, q0 + (nit - 1 - m) * rw);
  };
  if (nseq <= 1024) {
    // sequences by key count, descending (ties: lower index first), bitonic
    int lq, lk;
    key[tid] = tid < nseq ? (seq(tid, lq, lk), lk) : -1;
    idx[tid] = tid;
    __syncthreads();
    for (int k = 2; k <= 1024; k <<= 1)
      for (int j = k >> 1; j > 0; j >>= 1) {
        const int pj = tid ^ j;
        if (pj > tid) {
          const bool up = (tid & k) == 0;
          const bool partner_first = key[pj] > key[tid] || (key[pj] == key[tid] && idx[pj] < idx[tid]);
          if (up == partner_first) {
            const int tk = key[tid], ti = idx[tid];
            key[tid] = key[pj];
            idx[tid] = idx[pj];
            key[pj] = tk;
            idx[pj] = ti;
          }
        }
        __syncthreads();
      }
    const int s = idx[tid];
    const int nit = tid < nseq ? seq(s, lq, lk) : 0;
    const int incl = block_scan(nit);
    if (tid < nseq) emit(s, incl - nit);
    if (tid == 1023) *n_items = min(incl, cap_items);
  } else {
    for (int c0 = 0; c0 < nseq; c0 += 1024) {
      const int i = c0 + tid;
      int lq, lk;
      const int nit = i < nseq ? seq(i, lq, lk) : 0;
      const int incl = block_scan(nit);
      if (i < nseq) emit(i, base + incl - nit);
      __syncthreads();
      if (tid == 1023) base += incl;
      __syncthreads();
    }
    if (tid == 0) *n_items = min(base, cap_items);
  }
}

hipError_t prefill_varlen_prepare(const int32_t* cu_q, const int32_t* cu_k, int nseq, int total_q, int total_k,
                                  int rows_per_item, int4* items, int* n_items, int* counter, hipStream_t stream) {
  const int cap_items = (total_q + rows_per_item - 1) / rows_per_item + nseq;
  hipLaunchKernelGGL(prefill_varlen_prepare_kernel, dim3(1), dim3(1024), 0, stream, cu_q, cu_k, nseq, total_q,
                     total_k, rows_per_item, items, cap_items, n_items, counter);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

template <int DT, int H, int D, bool DENSE>
static hipError_t launch_variant(const PrefillParams& p, int grid, hipStream_t stream) {
  const size_t dyn = pf_dyn_bytes<DT, H, D>();
  if ((size_t)PfCfg<DT, H, D>::RW * p.sample_m * sizeof(float) > dyn) return hipErrorInvalidValue;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel<DT, H, D, DENSE>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((prefill_kernel<DT, H, D, DENSE>), dim3(grid), dim3(PfCfg<DT, H, D>::NT), dyn, stream, p);
  return hipGetLastError();
}

template <int DT, int H, int D>
static hipError_t launch_one(const PrefillParams& p, int grid, hipStream_t stream) {
  return p.out_dense ? launch_variant<DT, H, D, true>(p, grid, stream) : launch_variant<DT, H, D, false>(p, grid, stream);
}

// Every compiled (dtype, H, D) configuration.
#define DSA_PF_CONFIGS(X)                                                          \
  X(DSA_FP8_E4M3, 64, 128) X(DSA_FP8_E4M3, 64, 64) X(DSA_FP8_E4M3, 32, 128)        \
  X(DSA_FP8_E4M3, 32, 64) X(DSA_FP8_E4M3, 16, 128) X(DSA_FP8_E4M3, 16, 64)         \
  X(DSA_FP8_E4M3, 8, 128) X(DSA_FP8_E4M3, 8, 64) X(DSA_BF16, 64, 64)               \
  X(DSA_BF16, 32, 128) X(DSA_BF16, 32, 64) X(DSA_BF16, 16, 128) X(DSA_BF16, 16, 64) \
  X(DSA_BF16, 8, 128) X(DSA_BF16, 8, 64) X(DSA_BF16, 64, 128) X(DSA_FP8_E4M3, 128, 128)    \
  X(DSA_FP8_E4M3, 128, 64) X(DSA_BF16, 128, 128) X(DSA_BF16, 128, 64)

struct PfInfo {
  size_t static_lds;   // bytes of the kernel's static shared memory
  int tile_keys;       // keys per LDS tile
  int rows;            // query rows per work item
};

static bool pf_info(int dt, int H, int D, PfInfo* out) {
#define DSA_PF_INFO(DT_, H_, D_)                                                 \
  if (dt == DT_ && H == H_ && D == D_) {                                         \
    *out = PfInfo{sizeof(PfShared<DT_, H_, D_>), PfCfg<DT_, H_, D_>::TK, PfCfg<DT_, H_, D_>::RW};  \
    return true;                                                                 \
  }
  DSA_PF_CONFIGS(DSA_PF_INFO)
#undef DSA_PF_INFO
  return false;
}

int prefill_rows_per_item(int dt, int H, int D) {
  PfInfo info;
  return pf_info(dt, prefill_head_width(H), D, &info) ? info.rows : 0;
}

bool prefill_supported(int dt, int H, int D) {
  PfInfo info;
  return prefill_head_width(H) && pf_info(dt, prefill_head_width(H), D, &info);
}

// Keys per row sampled for the threshold estimate: the sampled scores of all
// rows of a work item live in dynamic LDS next to the kernel's static shared
// memory, at most 1024 per row, whole tiles only; fewer than 4 tiles disables
// the sample.
int prefill_sample_keys(int dt, int H, int D) {
  PfInfo info;
  if (!pf_info(dt, prefill_head_width(H), D, &info)) return 0;
  const size_t lds_limit = 160 * 1024;
  const int tk = info.tile_keys;
  const int rw = info.rows;
  if (info.static_lds >= lds_limit) return 0;
  int m = (int)((lds_limit - info.static_lds) / ((size_t)rw * sizeof(float)));
  m = m / tk * tk;
  if (m > 1024) m = 1024;
  return m >= 4 * tk ? m : 0;
}

// Candidate list capacity per row (workspace memory): 4*topk, at least topk
// plus 16 tiles, plus 2 tiles of slack, so that rows scored without a sample
// threshold (fewer than 4*topk keys) never need a compaction.  0 when the
// configuration is not built.
int prefill_list_capacity(int dt, int H, int D, int topk) {
  PfInfo info;
  if (!pf_info(dt, prefill_head_width(H), D, &info)) return 0;
  const size_t tk = (size_t)info.tile_keys;
  size_t cap = 4 * (size_t)topk;
  if (cap < (size_t)topk + 16 * tk) cap = (size_t)topk + 16 * tk;
  cap += 2 * tk;
  cap = (cap + 63) / 64 * 64;
  return (int)cap;
}

hipError_t prefill_launch(const PrefillParams& p, int dt, int H, int D, int grid, hipStream_t stream) {
  const long long n_dense = p.out_dense ? (long long)(p.L - p.q0) * p.L : 0;
  const int pg = n_dense ? 1024 : 1;
  hipLaunchKernelGGL(prefill_prepare_kernel, dim3(pg), dim3(256), 0, stream, p.counter, p.out_dense, n_dense);
  H = prefill_head_width(H);
#define DSA_PF_CASE(DT_, H_, D_) \
  if (dt == DT_ && H == H_ && D == D_) return launch_one<DT_, H_, D_>(p, grid, stream);
  DSA_PF_CONFIGS(DSA_PF_CASE)
#undef DSA_PF_CASE
  return hipErrorInvalidValue;
}

}  // namespace dsa
