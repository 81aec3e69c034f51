// Decode lightning indexer + top-k for gfx950.
//
// What is computed (Multi-layer Indexer abstract: at decode the indexer
// scores the whole cache of the sequence and keeps the k = 2048 best):
// sequence b has one bf16 query q[b] (H heads x D) at position len_b - 1; for
// every cached key s < len_b
//   score(b, s) = k_scale[b,s] * sum_h w[b,h] * ReLU(q[b,h] . k[b,s])
// and the min(k, len_b) best keys (score descending, index ascending) are
// written in ascending key order, padded with -1.
//
// Three launches:
// 1. decode_score_kernel streams the fp8 cache once.  A wave reads 32 whole
//    consecutive keys per step with 16-byte loads and keeps four steps in
//    flight.  Each lane owns one key column and the D/2 contiguous bytes of
//    its half of that key; fp8 is widened to bf16 exactly (e4m3 is a subset of
//    bf16) and the contraction runs on v_mfma_f32_32x32x16_bf16 with the heads
//    on the MFMA row dimension (q stays in registers).  The per-token fp32
//    scale multiplies the fp32 score (folding it into the bf16 operand would
//    not be exact).  Scores go to a workspace row, and each workgroup stores
//    its own 16-bit histograms of its keys' order-preserving images: 4096
//    fine bins (top 12 bits) and 256 coarse bins (top 8), written whole, so
//    nothing has to be cleared beforehand.  With a paged cache (a block
//    table of pages of 2^n >= 32 keys) each step lies in one page, whose id
//    each wave looks up once per step at the start.
// 2. decode_classify_kernel, several workgroups per sequence, each over a
//    16384-key slice: sums the coarse then the fine partial histograms to the
//    bin of the k-th score, marks the slice's keys of higher bins in a global
//    bitmap and gathers the keys of that bin as candidates.
// 3. decode_finalize_kernel, one workgroup per sequence: resolves the
//    candidates by radix select (ties to the lower index), marks the kept
//    ones and writes every marked key in ascending order.
// The kernel boundaries order the phases (no cross-workgroup fences).
#include "device_common.hpp"
#include "kernels.hpp"

namespace dsa {

namespace {

constexpr int DS_NT = 256;          // score kernel threads
constexpr int DS_NSUB = 64;         // 32-key steps per wave
static_assert(DS_NSUB <= 64, "paged lookup: one lane per step");
constexpr int DS_PF = 4;            // steps in flight per wave
constexpr int DS_KPB = (DS_NT / 64) * DS_NSUB * 32;   // keys per workgroup
constexpr int DS_MAXWG = 32;        // score workgroups per sequence at most (Lmax <= 262144)
constexpr int HBINS = 4096;         // fine bins: top 12 bits of the order-preserving key
constexpr int CBINS = 256;          // coarse bins: top 8 bits
constexpr int FPC = HBINS / CBINS;  // fine bins per coarse bin
constexpr int PW = HBINS / 2 + CBINS / 2;   // words of one score workgroup's packed histograms
constexpr int SL_NT = 1024;         // select threads
constexpr int SL_SLICE = 16384;     // scores per select workgroup
constexpr int SL_MAXG = 16;         // select workgroups per sequence at most (Lmax <= 262144)
constexpr int SL_CAP = 8192;        // candidate slots in LDS in the finalize kernel
constexpr int SL_SPEC = SL_CAP / SL_MAXG;   // candidates per slice read speculatively
constexpr int SL_MAXW = SL_MAXG * SL_SLICE / 32;   // bitmap words per sequence at most

// two e4m3 (bytes 2*HI, 2*HI+1 of src) -> two bf16, exact
template <bool HI>
__device__ __forceinline__ uint32_t cvt2(uint32_t src) {
  auto r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(src, 1.0f, HI);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ int seq_len(const DecodeParams& p, int b) {
  return min(max(p.lens[b], 0), p.Lmax);   // lengths outside [0, Lmax] are clamped
}

}  // namespace

template <int H, int D, bool PAGED>
__global__ void __launch_bounds__(DS_NT, 2) decode_score_kernel(DecodeParams p) {
  constexpr int MB = (H + 31) / 32;
  constexpr int KS = D / 16;              // bf16 MFMA steps along D
  constexpr int HALF = D / 2;             // fp8 bytes of one key half
  constexpr int NLD = HALF / 16;          // 16-byte loads per lane per 32-key step
  constexpr int CPR = D / 16;             // 16-byte chunks per key row
  constexpr int RPB = 256 / D;            // key rows per 256-byte bank sweep
  static_assert(32 * D == 1024 * NLD, "a step is NLD whole 1 KB loads");
  __shared__ uint32_t hist[HBINS];
  // per-wave transpose of one 32-key step: row r (a key), chunk c stored at
  // chunk position c ^ swz(r), swz(r) = (r / RPB) % CPR, so both the
  // row-contiguous writes and the per-key operand reads are conflict-free
  __shared__ __attribute__((aligned(16))) uint8_t ktr[DS_NT / 64][32 * D];
  // scores of the workgroup's keys; written out with 16-byte stores after the
  // loop so that no global store is in flight next to the MFMAs and loads
  __shared__ __attribute__((aligned(16))) float sc_stage[DS_KPB];

  const int b = blockIdx.y;
  const int len = seq_len(p, b);
  // Interleaved key mapping: step `sub` of wave w of workgroup x reads the
  // 32-key chunk (sub * nwg + x) * WAVES + w, so at any moment the workgroups
  // of a sequence sweep one contiguous region of its cache together.
  constexpr int WAVES = DS_NT / 64;
  const int nwg = gridDim.x;
  const int x = blockIdx.x;
  const int nchunk = (len + 31) >> 5;
  if (WAVES * x >= nchunk) return;
  // steps this workgroup needs (whole prefetch groups)
  const int nstep = min(DS_NSUB, ((nchunk - WAVES * x + WAVES * nwg - 1) / (WAVES * nwg) + DS_PF - 1) / DS_PF * DS_PF);

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int kh = lane >> 5;
  const int col = lane & 31;

  const uint8_t* cache_b = PAGED ? p.cache : p.cache + (size_t)b * p.Lmax * D;
  const float* ks_b = PAGED ? p.k_scale : p.k_scale + (size_t)b * p.Lmax;
  float* sc_b = p.scores + (size_t)b * p.ld;
  auto chunk_key = [&](int sub) { return 32 * ((sub * nwg + x) * WAVES + wave); };

  // q and w first: every later wait for them then leaves the cache prefetches
  // (issued after them) in flight
  // q operands: A row `col` of block mb is head 32*mb + col; lane half kh
  // holds d in [kh*D/2, (kh+1)*D/2), 8 consecutive values per MFMA step.
  v8bf qa[MB][KS];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int head = 32 * mb + col;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      v4i v = v4i{0, 0, 0, 0};
      if (head < H)
        v = *reinterpret_cast<const v4i*>(p.q + ((size_t)b * H + head) * D + kh * HALF + ks * 8);
      qa[mb][ks] = __builtin_bit_cast(v8bf, v);
    }
  }
  // result register j of block mb in this lane is head 32*mb + 8*(j/4) + 4*kh + j%4
  float wr[MB][16];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int head = 32 * mb + 8 * (j >> 2) + 4 * kh + (j & 3);
      wr[mb][j] = head < H ? bf16_to_f32(p.w[(size_t)b * H + head]) : 0.f;
    }
  // cache prefetch ring: step u lives in slot u % DS_PF.  Load i of a step
  // reads bytes [1024 i, 1024 i + 1024) of its 32 keys, 16 per lane (whole
  // keys, fully coalesced).  Loads are unconditional: a key past the end of
  // the sequence reads the last key instead (its score is never stored), so
  // no branch merges values into the ring registers and no wait is forced on
  // a load still in flight.
  v4i raw[DS_PF][NLD];
  float kss[DS_PF];
  // Paged cache: the 32 keys of a step (s0 a multiple of 32, pages of at
  // least 32 keys), clamped to the sequence, all lie in the page of
  // min(s0, len - 1).  Lane u of each wave looks up the page of its step u
  // once (nstep <= 64), so a fetch reads it from a register instead of
  // waiting for a table load.  Page ids outside [0, num_pages) are clamped
  // into it (no access leaves the page array).
  int step_page = 0;
  if constexpr (PAGED) {
    if (lane < nstep) {
      const int sb = min(chunk_key(lane), len - 1);
      step_page = p.block_table[(size_t)b * p.max_blocks + (sb >> p.page_shift)];
      step_page = min(max(step_page, 0), p.num_pages - 1);
    }
  }
  auto fetch = [&](int slot, int sub) {
    const int s0 = chunk_key(sub);
    const uint8_t* rows = cache_b;
    const float* kss_p = ks_b;
    int smask = 0;
    if constexpr (PAGED) {
      const int pg = __builtin_amdgcn_readlane(step_page, sub);
      rows = p.cache + ((size_t)pg << p.page_shift) * D;
      kss_p = p.k_scale + ((size_t)pg << p.page_shift);
      smask = (1 << p.page_shift) - 1;
    }
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int byte = 1024 * i + 16 * lane;
      const int r = byte / D;
      int s = min(s0 + r, len - 1);
      if constexpr (PAGED) s &= smask;
      raw[slot][i] = *reinterpret_cast<const v4i*>(rows + (size_t)s * D + byte % D);
    }
    int sk = min(s0 + col, len - 1);
    if constexpr (PAGED) sk &= smask;
    kss[slot] = kss_p[sk];
  };
  uint8_t* tr = ktr[wave];
  // this lane's operand chunks: key `col`, chunks kh*NLD + i of its row
  const int rswz = (col / RPB) % CPR;
#pragma unroll
  for (int u = 0; u < DS_PF; ++u) fetch(u, u);

  for (int i = tid; i < HBINS; i += DS_NT) hist[i] = 0u;
  __syncthreads();

  // the ring is unrolled inside a rolled loop; with unconditional loads every
  // slot keeps its registers across iterations
#pragma unroll 1
  for (int g = 0; g < nstep; g += DS_PF) {
#pragma unroll
    for (int u = 0; u < DS_PF; ++u) {
      const int sub = g + u;
      const int s0 = chunk_key(sub);
      {
        // through the wave's LDS transpose into per-key operand order
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
          const int byte = 1024 * i + 16 * lane;
          const int r = byte / D, c = (byte % D) / 16;
          *reinterpret_cast<v4i*>(tr + r * D + 16 * (c ^ ((r / RPB) % CPR))) = raw[u][i];
        }
        const float cks = kss[u];
        fetch(u, min(sub + DS_PF, nstep - 1));   // past the end: harmless reload
        wave_lds_sync();
        v4i cur[NLD];
#pragma unroll
        for (int i = 0; i < NLD; ++i)
          cur[i] = *reinterpret_cast<const v4i*>(tr + col * D + 16 * ((kh * NLD + i) ^ rswz));
        wave_lds_sync();   // every lane has read before the next step overwrites

        v16f acc[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[mb] = v16f{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          // widen 8 fp8 (half of a 16-byte load) into one bf16 operand, just in time
          const uint32_t d0 = (uint32_t)cur[ks >> 1][2 * (ks & 1)];
          const uint32_t d1 = (uint32_t)cur[ks >> 1][2 * (ks & 1) + 1];
          const v8bf bop = __builtin_bit_cast(v8bf, v4i{(int)cvt2<false>(d0), (int)cvt2<true>(d0),
                                                        (int)cvt2<false>(d1), (int)cvt2<true>(d1)});
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) acc[mb] = mfma_bf16(qa[mb][ks], bop, acc[mb]);
        }
        float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int j = 0; j < 16; ++j) part[j & 3] = fmaf(wr[mb][j], fmaxf(acc[mb][j], 0.f), part[j & 3]);
        float tot = (part[0] + part[1]) + (part[2] + part[3]);
        tot += __shfl_xor(tot, 32);          // the other half holds the other heads
        const float score = tot * cks;
        const int s = s0 + col;
        if (kh == 0 && s < len) {
          sc_stage[sub * (32 * WAVES) + wave * 32 + col] = score;
          atomicAdd(&hist[ordered_key(score) >> 20], 1u);
        }
      }
    }
  }
  __syncthreads();
  // each step wrote 32*WAVES consecutive keys; score rows are 64-float
  // aligned (ld), so the 16-byte stores are aligned
  for (int i = tid; i < nstep * 8 * WAVES; i += DS_NT) {
    const int sub = i / (8 * WAVES), q4 = i % (8 * WAVES);
    const int s = 32 * WAVES * (sub * nwg + x) + 4 * q4;
    const v4i v = reinterpret_cast<const v4i*>(sc_stage)[i];
    if (s + 3 < len) {
      *reinterpret_cast<v4i*>(sc_b + s) = v;
    } else {
      for (int e = 0; e < 4; ++e)
        if (s + e < len) sc_b[s + e] = __int_as_float(v[e]);
    }
  }
  // this workgroup's histograms, stored whole as 16-bit counts (a workgroup
  // scores at most DS_KPB < 65536 keys): no atomics, nothing to clear.
  // Words [0, HBINS/2): the fine bins in pairs; [HBINS/2, PW): the coarse
  // bins (sums of FPC consecutive fine bins) in pairs.
  uint32_t* gh = p.hist + ((size_t)b * nwg + x) * PW;
  for (int i = tid; i < HBINS / 8; i += DS_NT) {
    const v4i lo = reinterpret_cast<const v4i*>(hist)[2 * i];
    const v4i hi = reinterpret_cast<const v4i*>(hist)[2 * i + 1];
    reinterpret_cast<v4i*>(gh)[i] = v4i{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16), hi[0] | (hi[1] << 16),
                                        hi[2] | (hi[3] << 16)};
  }
  for (int i = tid; i < CBINS / 2; i += DS_NT) {
    uint32_t c[2] = {0u, 0u};
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int q = 0; q < FPC / 4; ++q) {
        const v4i t = reinterpret_cast<const v4i*>(hist)[(2 * i + h) * (FPC / 4) + q];
        c[h] += (uint32_t)(t[0] + t[1] + t[2] + t[3]);
      }
    gh[HBINS / 2 + i] = c[0] | (c[1] << 16);
  }
}

// ---------------------------------------------------------------------------
// select: the classify kernel finds the bin of the k-th score and sorts each
// slice of SL_SLICE scores into selected keys and candidates; the finalize
// kernel resolves the candidates and writes the ascending top-k
// ---------------------------------------------------------------------------

namespace {

static_assert(DS_KPB < 65536, "16-bit partial histograms");

struct SelShared {
  uint32_t hist[HBINS];               // sequence histogram of the top 12 key bits
  uint32_t hist8[256];
  int wtot[SL_NT / 64];
  int coff[SL_MAXG + 1];              // candidate offsets of the slices
  int bc[4];
  int ncand;
};

// exclusive scan of v over the workgroup; *total gets the sum
__device__ int sl_scan(int v, SelShared& sh, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int incl = wave_incl_sum(v);
  if (lane == 63) sh.wtot[wave] = incl;
  __syncthreads();
  int pre = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < SL_NT / 64; ++w) {
    const int x = sh.wtot[w];
    pre += (w < wave) ? x : 0;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return pre + incl - v;
}

}  // namespace

__global__ void __launch_bounds__(SL_NT) decode_classify_kernel(DecodeParams p, int nwg) {
  __shared__ SelShared sh;
  const int g = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = seq_len(p, b);
  const int k = p.topk;
  int* out = p.out_idx + (size_t)b * k;
  float* osc = p.out_score ? p.out_score + (size_t)b * k : nullptr;
  const float* sc = p.scores + (size_t)b * p.ld;

  if (n <= k) {                       // every key is kept
    if (g == 0)
      for (int j = tid; j < k; j += SL_NT) {
        out[j] = j < n ? j : -1;
        if (osc) osc[j] = j < n ? sc[j] : -__builtin_inff();
      }
    return;
  }
  const int nslice = (n + SL_SLICE - 1) / SL_SLICE;
  if (g >= nslice) return;
  const int nwmax = (p.Lmax + 31) >> 5;
  uint32_t* gbm = p.bitmap + (size_t)b * nwmax;
  uint32_t* gkey = p.cand_key + (size_t)b * p.Lmax;
  int* gidx = p.cand_idx + (size_t)b * p.Lmax;

  // 1. the coarse histograms of the active score workgroups (those that had
  //    keys), then this slice's scores (a float4 per lane and load, 256
  //    consecutive scores per wave and load; the row holds at least 4 nq
  //    floats): loads complete in issue order, so the histogram work below
  //    does not wait for the scores
  const int nchunk = (n + 31) >> 5;
  const int nact = min(nwg, (nchunk + DS_NT / 64 - 1) / (DS_NT / 64));
  const uint32_t* ph = p.hist + (size_t)b * nwg * PW;
  constexpr int CW = CBINS / 2;       // coarse words per partial
  constexpr int PS = SL_NT / CW;      // partials read side by side
  constexpr int CU = (DS_MAXWG + PS - 1) / PS;
  uint32_t ct[CU];
#pragma unroll
  for (int u = 0; u < CU; ++u) ct[u] = ph[(size_t)min(tid / CW + PS * u, nact - 1) * PW + HBINS / 2 + tid % CW];
  const int s0 = g * SL_SLICE;
  const int nq = (n + 3) >> 2;
  constexpr int SU = SL_SLICE / (4 * SL_NT);
  v4f v[SU];
#pragma unroll
  for (int u = 0; u < SU; ++u) {
    const int gi = (SL_NT / 64) * u + wave;
    v[u] = reinterpret_cast<const v4f*>(sc)[min((s0 >> 2) + 64 * gi + lane, nq - 1)];
  }
  {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int u = 0; u < CU; ++u)
      if (tid / CW + PS * u < nact) {
        lo += ct[u] & 0xFFFFu;
        hi += ct[u] >> 16;
      }
    if (tid < CBINS) sh.hist[tid] = 0u;
    if (tid < FPC) sh.hist8[tid] = 0u;
    if (tid == 0) sh.ncand = 0;
    __syncthreads();
    if (lo) atomicAdd(&sh.hist[2 * (tid % CW)], lo);
    if (hi) atomicAdd(&sh.hist[2 * (tid % CW) + 1], hi);
    __syncthreads();
  }

  // 2. bin d* of the k-th score and the number of keys above it: first the
  //    coarse bin, then its FPC fine bins (read from the partials only there)
  {
    const int hv = tid < CBINS ? (int)sh.hist[tid] : 0;
    int tot;
    const int pre = sl_scan(hv, sh, &tot);
    const int ab = tot - pre - hv;     // keys in higher coarse bins
    if (tid < CBINS && ab < k && ab + hv >= k) {
      sh.bc[0] = tid;
      sh.bc[1] = ab;
    }
    __syncthreads();
    const int cstar = sh.bc[0];
    if (tid < (FPC / 2) * nact) {
      const uint32_t t = ph[(size_t)(tid / (FPC / 2)) * PW + (FPC / 2) * cstar + tid % (FPC / 2)];
      if (t & 0xFFFFu) atomicAdd(&sh.hist8[2 * (tid % (FPC / 2))], t & 0xFFFFu);
      if (t >> 16) atomicAdd(&sh.hist8[2 * (tid % (FPC / 2)) + 1], t >> 16);
    }
    __syncthreads();
    if (wave == 0) {
      const int h = lane < FPC ? (int)sh.hist8[lane] : 0;
      int incl = h;                     // keys in fine bins lane.. of the coarse bin
#pragma unroll
      for (int o = 1; o < FPC; o <<= 1) {
        const int t = __shfl_down(incl, o);
        if (lane + o < FPC) incl += t;
      }
      const int ab2 = sh.bc[1] + incl - h;
      if (lane < FPC && ab2 < k && ab2 + h >= k) {
        sh.bc[2] = FPC * cstar + lane;
        sh.bc[3] = ab2;
      }
    }
    __syncthreads();
  }
  const uint32_t dstar = (uint32_t)sh.bc[2];

  // 3. classify the slice: keys of higher bins are marked in the global
  //    bitmap (eight lanes OR their four bits into one word), keys of bin d*
  //    go to this slice's candidate region
  {
    uint32_t cnd[SU];
    uint32_t key[SU][4];
#pragma unroll
    for (int u = 0; u < SU; ++u) {
      const int j0 = s0 + 256 * ((SL_NT / 64) * u + wave) + 4 * lane;
      uint32_t selb = 0;
      cnd[u] = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool valid = j0 + e < n;
        key[u][e] = ordered_key(v[u][e]);
        const uint32_t dg = key[u][e] >> 20;
        selb |= (uint32_t)(valid && dg > dstar) << e;
        cnd[u] |= (uint32_t)(valid && dg == dstar) << e;
      }
      uint32_t word = selb << (4 * (lane & 7));
      word |= (uint32_t)__shfl_xor((int)word, 1);
      word |= (uint32_t)__shfl_xor((int)word, 2);
      word |= (uint32_t)__shfl_xor((int)word, 4);
      if ((lane & 7) == 0 && j0 < n) gbm[j0 >> 5] = word;
    }
    // compaction: one LDS atomic per wave
    uint64_t me[SU][4];
    int tot = 0;
#pragma unroll
    for (int u = 0; u < SU; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        me[u][e] = ballot64((cnd[u] >> e) & 1u);
        tot += __popcll(me[u][e]);
      }
    if (tot) {                        // uniform
      int c0 = 0;
      if (lane == 0) c0 = atomicAdd(&sh.ncand, tot);
      c0 = __shfl(c0, 0);
#pragma unroll
      for (int u = 0; u < SU; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if ((cnd[u] >> e) & 1u) {
            const int c = c0 + lanes_below(me[u][e]);
            gkey[s0 + c] = key[u][e];
            gidx[s0 + c] = s0 + 256 * ((SL_NT / 64) * u + wave) + 4 * lane + e;
          }
          c0 += __popcll(me[u][e]);
        }
    }
  }
  __syncthreads();
  if (tid == 0) {
    p.cand_cnt[(size_t)b * SL_MAXG + g] = sh.ncand;
    if (g == 0) p.cut[b] = int2{(int)dstar, sh.bc[3]};
  }
}

// One workgroup per sequence, after the classify kernel: resolve the k-th
// score among the candidates and write the ascending top-k.
__global__ void __launch_bounds__(SL_NT) decode_finalize_kernel(DecodeParams p) {
  extern __shared__ uint32_t dyn[];
  __shared__ SelShared sh;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int n = seq_len(p, b);
  const int k = p.topk;
  if (n <= k) return;                 // written by the classify kernel
  int* out = p.out_idx + (size_t)b * k;
  float* osc = p.out_score ? p.out_score + (size_t)b * k : nullptr;
  const float* sc = p.scores + (size_t)b * p.ld;
  const int nslice = (n + SL_SLICE - 1) / SL_SLICE;
  const int nwmax = (p.Lmax + 31) >> 5;
  const uint32_t* gbm = p.bitmap + (size_t)b * nwmax;
  const uint32_t* gkey = p.cand_key + (size_t)b * p.Lmax;
  const int* gidx = p.cand_idx + (size_t)b * p.Lmax;
  const int2 cut = p.cut[b];
  const uint32_t dstar = (uint32_t)cut.x;

  // 4. one round of loads: the bitmap, the candidate counts, and the first
  //    SL_SPEC entries of every slice's candidate region (a count above
  //    SL_SPEC, which is rare, sends every pass below to global memory)
  const int nw = (n + 31) >> 5;       // bitmap words
  uint32_t* bm = dyn;                 // selected keys
  uint32_t* tb = dyn + nw;            // keys tied with the k-th score
  uint32_t* lkey = dyn + 2 * nw;      // slice x's first entries at x * SL_SPEC
  int* lidx = reinterpret_cast<int*>(lkey + SL_CAP);
  {
    // every load is issued before any result is stored
    constexpr int BR = SL_MAXW / SL_NT;           // bitmap words per thread at most
    constexpr int CR = SL_CAP / SL_NT;            // candidate slots per thread
    const int cnt = tid < nslice ? p.cand_cnt[(size_t)b * SL_MAXG + tid] : 0;
    uint32_t bw[BR], ck[CR];
    int cx[CR];
#pragma unroll
    for (int r = 0; r < BR; ++r) bw[r] = gbm[min(tid + SL_NT * r, nw - 1)];
#pragma unroll
    for (int r = 0; r < CR; ++r) {
      const int c = tid + SL_NT * r;
      const int e = min((c / SL_SPEC) * SL_SLICE + c % SL_SPEC, p.Lmax - 1);
      if (c < nslice * SL_SPEC) {
        ck[r] = gkey[e];
        cx[r] = gidx[e];
      }
    }
    if (tid < nslice) sh.coff[tid] = cnt;
#pragma unroll
    for (int r = 0; r < BR; ++r)
      if (tid + SL_NT * r < nw) {
        bm[tid + SL_NT * r] = bw[r];
        tb[tid + SL_NT * r] = 0u;
      }
#pragma unroll
    for (int r = 0; r < CR; ++r)
      if (tid + SL_NT * r < nslice * SL_SPEC) {
        lkey[tid + SL_NT * r] = ck[r];
        lidx[tid + SL_NT * r] = cx[r];
      }
    if (tid == 0) sh.ncand = 0;       // ties with the k-th key
    __syncthreads();
  }
  bool spill = false;
  for (int x = 0; x < nslice; ++x) spill |= sh.coff[x] > SL_SPEC;
  // calls body(key, index) for every candidate
  auto for_cand = [&](auto body) {
    if (!spill) {
      for (int c = tid; c < nslice * SL_SPEC; c += SL_NT)
        if (c % SL_SPEC < sh.coff[c / SL_SPEC]) body(lkey[c], lidx[c]);
    } else {
      for (int x = 0; x < nslice; ++x)
        for (int i = tid; i < sh.coff[x]; i += SL_NT) body(gkey[x * SL_SLICE + i], gidx[x * SL_SLICE + i]);
    }
  };

  // 5. exact k-th key among the candidates (they share the top 12 bits):
  //    two rounds of 1024 bins, one per thread
  int need = k - cut.y;               // keys still to take from bin d* (>= 1)
  uint32_t prefix = dstar << 20;
  uint32_t pmask = 0xFFF00000u;
  static_assert(SL_NT == 1024, "one radix bin per thread");
#pragma unroll 1
  for (int shift = 10; shift >= 0; shift -= 10) {
    sh.hist[tid] = 0u;
    __syncthreads();
    for_cand([&](uint32_t key, int) {
      if ((key & pmask) == prefix) atomicAdd(&sh.hist[(key >> shift) & 1023u], 1u);
    });
    __syncthreads();
    const int hv = (int)sh.hist[tid];
    int t2;
    const int pre = sl_scan(hv, sh, &t2);
    const int ab = t2 - pre - hv;      // entries in higher bins
    if (ab < need && ab + hv >= need) {
      sh.bc[2] = tid;
      sh.bc[3] = ab;
    }
    __syncthreads();
    prefix |= (uint32_t)sh.bc[2] << shift;
    pmask |= 1023u << shift;
    need -= sh.bc[3];
  }
  const uint32_t kstar = prefix;
  for_cand([&](uint32_t key, int j) {
    if (key > kstar) {
      atomicOr(&bm[j >> 5], 1u << (j & 31));
    } else if (key == kstar) {
      atomicOr(&tb[j >> 5], 1u << (j & 31));
      atomicAdd(&sh.ncand, 1);
    }
  });
  __syncthreads();

  // 6. ties with the k-th score: when more than `need` keys tie, the `need`
  //    lowest indices (otherwise every tied key is taken)
  const int wpt = (nw + SL_NT - 1) / SL_NT;   // bitmap words per thread, contiguous
  if (sh.ncand == need) {             // uniform
    for (int i = 0; i < wpt; ++i) {
      const int wd = tid * wpt + i;
      if (wd < nw) bm[wd] |= tb[wd];
    }
  } else {
    int c = 0;
    for (int i = 0; i < wpt; ++i) {
      const int wd = tid * wpt + i;
      if (wd < nw) c += __popc(tb[wd]);
    }
    int t3;
    int before = sl_scan(c, sh, &t3);
    for (int i = 0; i < wpt; ++i) {
      const int wd = tid * wpt + i;
      if (wd >= nw) break;
      uint32_t x = tb[wd];
      while (x) {
        const int bpos = __ffs(x) - 1;
        x &= x - 1;
        if (before < need) bm[wd] |= 1u << bpos;
        ++before;
      }
    }
  }

  // 7. the selection in ascending key order (each thread's words are its own)
  {
    int c = 0;
    for (int i = 0; i < wpt; ++i) {
      const int wd = tid * wpt + i;
      if (wd < nw) c += __popc(bm[wd]);
    }
    int t4;
    int pos = sl_scan(c, sh, &t4);
    for (int i = 0; i < wpt; ++i) {
      const int wd = tid * wpt + i;
      if (wd >= nw) break;
      uint32_t x = bm[wd];
      while (x) {
        const int bpos = __ffs(x) - 1;
        x &= x - 1;
        const int j = wd * 32 + bpos;
        if (pos < k) {
          out[pos] = j;
          if (osc) osc[pos] = sc[j];
        }
        ++pos;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

static int score_workgroups(int Lmax) { return (Lmax + DS_KPB - 1) / DS_KPB; }
static int select_workgroups(int Lmax) { return (Lmax + SL_SLICE - 1) / SL_SLICE; }

size_t decode_select_lds_bytes(int Lmax) {
  const size_t nw = ((size_t)Lmax + 31) / 32;
  return 2 * nw * sizeof(uint32_t) + (size_t)SL_CAP * (sizeof(uint32_t) + sizeof(int));
}

bool decode_supported(int H, int D, int Lmax) {
  if (!(H == 16 || H == 32 || H == 64)) return false;
  if (D != 64 && D != 128) return false;
  if (select_workgroups(Lmax) > SL_MAXG || score_workgroups(Lmax) > DS_MAXWG) return false;
  return decode_select_lds_bytes(Lmax) + sizeof(SelShared) <= 160 * 1024;
}

DecodeWsSizes decode_ws_sizes(int Lmax) {
  DecodeWsSizes z;
  z.hist_words = (size_t)score_workgroups(Lmax) * PW;
  z.bitmap_words = ((size_t)Lmax + 31) / 32;
  z.cand_cnt = SL_MAXG;
  return z;
}

template <int H, int D>
static void launch_score(const DecodeParams& p, hipStream_t stream) {
  dim3 grid(score_workgroups(p.Lmax), p.B);
  if (p.block_table) hipLaunchKernelGGL((decode_score_kernel<H, D, true>), grid, dim3(DS_NT), 0, stream, p);
  else hipLaunchKernelGGL((decode_score_kernel<H, D, false>), grid, dim3(DS_NT), 0, stream, p);
}

hipError_t decode_launch(const DecodeParams& p, int H, int D, hipStream_t stream) {
  if (H == 64 && D == 128) launch_score<64, 128>(p, stream);
  else if (H == 64 && D == 64) launch_score<64, 64>(p, stream);
  else if (H == 32 && D == 128) launch_score<32, 128>(p, stream);
  else if (H == 32 && D == 64) launch_score<32, 64>(p, stream);
  else if (H == 16 && D == 128) launch_score<16, 128>(p, stream);
  else if (H == 16 && D == 64) launch_score<16, 64>(p, stream);
  else return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_classify_kernel, dim3(select_workgroups(p.Lmax), p.B), dim3(SL_NT), 0, stream, p,
                     score_workgroups(p.Lmax));
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = decode_select_lds_bytes(p.Lmax);
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(decode_finalize_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_finalize_kernel, dim3(p.B), dim3(SL_NT), lds, stream, p);
  return hipGetLastError();
}

}  // namespace dsa
