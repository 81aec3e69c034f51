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
// Two launches:
// 1. decode_score_kernel streams the fp8 cache once.  A workgroup owns up to
//    8192 keys of one sequence on average (32-key steps interleaved with the
//    other workgroups of the sequence, the last quarter claimed from a
//    shared pool), at most 10240.  A wave reads 32 whole consecutive keys per
//    step with 16-byte buffer loads (keys past the sequence read as 0 at the
//    buffer's record limit) and keeps four steps in flight; a per-wave LDS
//    transpose gives each lane one key column.  The contraction runs on the
//    fp8 matrix cores: the bf16 query is split into two e4m3 limbs with e8m0
//    scales per block of 32 dimensions (exact unless a block spans more than
//    2^14 in magnitude, else within 2^-22 of the block's largest value),
//    stacked along K, so the keys are used as they are stored.  ReLU and the
//    head-weighted sum follow in fp32, then the per-token k_scale.  Scores
//    stay in LDS with a 4096-bin histogram of their order-preserving images
//    (top 12 bits).  At the end the workgroup keeps its own min(k, n) best
//    keys plus the rest of their boundary bin and writes them with their
//    indices, grouped by bin from the highest: every key of the sequence's
//    top k is among its workgroup's top k, so these lists hold the whole
//    answer.  Its 16-bit histograms go out beside them: all 256 coarse
//    bins, and the 4096 fine bins from the coarse bin of its cut up (the
//    select reads none below a list's cut).
// 2. decode_select_kernel, one workgroup per sequence: sums the coarse then
//    the fine histograms of the sequence's workgroups to the bin of the k-th
//    score, reads from every list only its prefix of bins at or above that
//    bin (into registers), resolves the boundary bin exactly (ties to the
//    lower index) and writes the selection in ascending key order through
//    an LDS bitmap.
// With a paged cache (a block table of pages of 2^n >= 32 keys) each step
// lies in one page, whose id each wave looks up once, at the start.
// The kernel boundary orders the phases (no cross-workgroup fences).
#include <mutex>

#include "device_common.hpp"
#include "kernels.hpp"

namespace dsa {

namespace {

constexpr int DS_NT = 256;          // score kernel threads
constexpr int DS_WAVES = DS_NT / 64;
constexpr int DS_NSUB = 64;         // 32-key steps per wave on average (the static map's unit)
constexpr int DS_CAP = 80;          // 32-key steps a wave can hold (room to take pool chunks)
constexpr int DS_PF = 4;            // steps in flight per wave
constexpr int DS_KPB = DS_WAVES * DS_NSUB * 32;   // keys per workgroup on average (sets the grid)
constexpr int DS_KCAP = DS_WAVES * DS_CAP * 32;   // keys a workgroup can hold
constexpr int DS_MAXWG = 32;        // score workgroups per sequence at most (Lmax <= 262144)
constexpr int DS_MAXPOOL = 1024;    // pool chunks per sequence at most, paged cache (pages in LDS)
constexpr int HBINS = 4096;         // fine bins: top 12 bits of the order-preserving key
constexpr int CBINS = 256;          // coarse bins: top 8 bits
constexpr int FPC = HBINS / CBINS;  // fine bins per coarse bin
constexpr int PW = HBINS / 2 + CBINS / 2;   // words of one score workgroup's packed histograms
constexpr int SL_NT = 1024;         // select threads

static_assert(DS_KCAP < 65536, "16-bit partial histograms");
static_assert(DS_NT * 16 == HBINS, "score kernel tail: 16 bins per thread");

__device__ __forceinline__ int seq_len(const DecodeParams& p, int b) {
  return min(max(p.lens[b], 0), p.Lmax);   // lengths outside [0, Lmax] are clamped
}

typedef uint32_t v2u __attribute__((ext_vector_type(2)));

// Buffer resource of `bytes` bytes at `base` (gfx9 descriptor word 3):
// loads at offsets past `bytes` return 0 without touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// fp8 MFMA with per-lane A block scales, byte KK of scale_a.  On gfx950 the
// e8m0 scale that lane (row, half c) passes applies to bytes [16c, 16c + 16)
// of both lanes of that row: one 32-element block of K.
template <int KK>
__device__ __forceinline__ v16f mfma_kk(v8i a, v8i b, v16f c, int scale_a) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, KK, scale_a, 0, 127);
}

// tag of a call's pool counter: a 32-bit mix of the launch nonce, the
// sequence's generation word and the sequence index
__device__ __forceinline__ uint32_t pool_tag(uint32_t nonce, uint32_t gen, int b) {
  uint32_t h = nonce ^ (gen * 0x9E3779B9u) ^ ((uint32_t)b * 0x85EBCA6Bu);
  h ^= h >> 16;
  h *= 0x7FEB352Du;
  h ^= h >> 15;
  h *= 0x846CA68Bu;
  h ^= h >> 16;
  return h;
}

__device__ __forceinline__ int score_grid_nwg(int Lmax) { return (Lmax + DS_KPB - 1) / DS_KPB; }

// Workgroup -> (sequence, its workgroup index).  Workgroups go to the 8 XCDs
// round-robin and fill the CUs in dispatch order, so when nwg is a multiple
// of 8 the map gives every sequence workgroups on every XCD, early and late
// in the dispatch order alike (XCD = L % 8; the m-th workgroup of an XCD
// serves sequence m % B).  Otherwise a sequence's workgroups are consecutive.
__device__ __forceinline__ void score_block(int L, int B, int nwg, int& b, int& x) {
  if (nwg % 8 == 0) {
    const int xcd = L & 7, m = L >> 3;
    b = m % B;
    x = (m / B) * 8 + xcd;
  } else {
    b = L / nwg;
    x = L % nwg;
  }
}

constexpr float LIMB_MIN = 7.8886091e-31f;     // 2^-100: a smaller block maximum drops the block

// e8m0 exponent e with m 2^-e in (224, 448], for m >= LIMB_MIN
__device__ __forceinline__ int limb_exp(float m) {
  const uint32_t mu = __float_as_uint(m);
  return (int)((mu >> 23) & 255u) - 127 - ((mu & 0x7FFFFFu) <= 0x600000u ? 8 : 7);
}

}  // namespace

// Two workgroups per CU, except at H = 128, whose query limbs alone take
// 128 registers: one wave per SIMD.
template <int H, int D, bool PAGED>
__global__ void __launch_bounds__(DS_NT, H > 64 ? 1 : 2) decode_score_kernel(DecodeParams p) {
  constexpr int MB = (H + 31) / 32;
  constexpr int KS = D / 64;              // fp8 MFMA steps along D
  constexpr int NK = 2 * KS;              // with the two limbs of q stacked along K
  constexpr int HALF = D / 2;             // fp8 bytes of one key half
  constexpr int NLD = HALF / 16;          // 16-byte loads per lane per 32-key step
  constexpr int CPR = D / 16;             // 16-byte chunks per key row
  constexpr int RPB = 256 / D;            // key rows per 256-byte bank sweep
  static_assert(32 * D == 1024 * NLD, "a step is NLD whole 1 KB loads");
  static_assert(NK <= 4, "limb scale bytes");
  __shared__ uint32_t hist[HBINS];
  // per-wave transpose of one 32-key step: row r (a key), chunk c stored at
  // chunk position c ^ swz(r), swz(r) = (r / RPB) % CPR, so both the
  // row-contiguous writes and the per-key operand reads are conflict-free;
  // at the start, the query's limbs in operand order
  __shared__ __attribute__((aligned(16))) uint8_t ktr[DS_WAVES][32 * D];
  // order-preserving keys of the workgroup's scores; at the start, the
  // limbs' scales
  __shared__ __attribute__((aligned(16))) float sc_stage[DS_KCAP];
  __shared__ int sh_cut[2];
  // the k_scale of the step being scored, per wave (through LDS, so that
  // the load's register is free again before the next load into it)
  __shared__ float kst[DS_WAVES][32];
  // chunk read at each local step of each wave (-1: none), and the number
  // of steps each wave read, for the tail
  __shared__ int step_chunk[DS_WAVES][DS_CAP];
  __shared__ int wave_steps[DS_WAVES];
  // paged cache: the page of every pool chunk
  __shared__ int pool_page[PAGED ? DS_MAXPOOL : 1];

  const int nwg = score_grid_nwg(p.Lmax);
  int b, x;
  score_block(blockIdx.x, p.B, nwg, b, x);
  const int len = __builtin_amdgcn_readfirstlane(seq_len(p, b));   // uniform: scalar descriptors
  // Interleaved key mapping: static step `sub` of wave w of workgroup x reads
  // the 32-key chunk (sub * nwg + x) * WAVES + w, so at any moment the
  // workgroups of a sequence sweep one contiguous region of its cache.
  const int nchunk = (len + 31) >> 5;
  if (DS_WAVES * x >= nchunk) return;     // the select kernel counts only active workgroups
  // Every wave of the sequence reads its first S steps from the interleaved
  // static map (S a multiple of the ring depth: about half of the chunks in
  // all; with a paged cache about 3/4, and at least all but DS_MAXPOOL, whose
  // pages are looked up in advance); the remaining chunks form a pool that
  // the waves claim, a ring's worth at a time, from a shared counter once
  // their static steps are issued, so that waves on slower parts of the
  // chip, or dispatched later, end no later than the others.  A wave holds
  // up to DS_CAP steps, more than the average DS_NSUB.
  constexpr int SNUM = PAGED ? 3 : 1, SDEN = PAGED ? 4 : 2;
  const int S = max((nchunk * SNUM / SDEN) / (DS_WAVES * nwg) / DS_PF * DS_PF,
                    PAGED ? (max(nchunk - DS_MAXPOOL, 0) + DS_WAVES * nwg * DS_PF - 1) / (DS_WAVES * nwg * DS_PF) * DS_PF
                          : 0);
  const int nstat = S * DS_WAVES * nwg;
  const int npool = nchunk - nstat;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int kh = lane >> 5;
  const int col = lane & 31;

  // static step sub < S reads chunk (sub * nwg + x) * WAVES + wave
  auto static_chunk = [&](int sub) { return (sub * nwg + x) * DS_WAVES + wave; };

  // Pool counter of the sequence: a 64-bit word, claim count in the low
  // half and, in the high half, the tag of the call that owns it.  The tag
  // mixes the host's per-launch nonce with the sequence's generation word,
  // which the select kernel advances after every call, so a word left by an
  // earlier call (or arbitrary workspace bytes, except with probability
  // 2^-32) carries another tag; the first claimer that sees one re-tags it
  // with a compare-and-swap and count 0.  Nothing needs clearing.
  DecodeHdr* hdr = p.hdr + b;
  const uint32_t tag = (uint32_t)__builtin_amdgcn_readfirstlane((int)pool_tag(p.nonce, hdr->gen, b));
  unsigned long long* pool = &hdr->pool;
  // a claim's old counter value -> the first pool entry of its batch of
  // DS_PF entries (lane 0 only)
  auto take = [&](unsigned long long old) -> uint32_t {
    if ((uint32_t)(old >> 32) != tag) {          // stale: re-tag (rare)
      bool mine = false;
      while ((uint32_t)(old >> 32) != tag) {
        const unsigned long long want = old + DS_PF;   // the claim already added DS_PF
        const unsigned long long seen =
            atomicCAS(pool, want, (unsigned long long)tag << 32 | (unsigned long long)DS_PF);
        if (seen == want) {
          mine = true;                             // claimed entries 0 .. DS_PF - 1
          break;
        }
        old = atomicAdd(pool, (unsigned long long)DS_PF);
      }
      // settle this path's atomics here, so that the register tracking of
      // the common path does not inherit them as pending
      __builtin_amdgcn_s_waitcnt(0);
      if (mine) return 0u;
    }
    return (uint32_t)old;
  };

  // cache prefetch ring: step u lives in slot u % DS_PF.  Load i of a step
  // reads bytes [1024 i, 1024 i + 1024) of its 32 keys, 16 per lane (whole
  // keys, fully coalesced); the record limit turns keys past the sequence
  // (or past the page's keys of the sequence) into zeros, whose scores are
  // never stored.
  v4i raw[DS_PF][NLD];
  float kss[DS_PF];
  // Paged cache: the 32 keys of a step (s0 a multiple of 32, pages of at
  // least 32 keys) lie in one page; lane u of each wave looks up the page of
  // its static step u once (at most 56 of them), and the pool chunks' pages
  // go to LDS.  Page ids outside [0, num_pages) are
  // clamped into it (no access leaves the page array).
  // The query block and head weights are loaded first: loads return in
  // order, so the limb arithmetic below waits only for these, not for the
  // cache steps issued after them.
  // Block (head, ks, c) of the query holds the 32 dims
  // {h HALF + 32 ks + 16 c + i : h < 2, i < 16}, which MFMA step ks reads
  // from bytes [16c, 16c + 16) of both lane halves; thread blk owns block blk.
  constexpr int NBLK = 32 * MB * KS * 2;
  constexpr int QB = (NBLK + DS_NT - 1) / DS_NT;   // query blocks per thread: block tid + DS_NT j
  v4i qraw[QB][2][2];
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    const int blk = tid + DS_NT * j;
    const int qhead = blk / (KS * 2), qks = (blk >> 1) % KS, qc = blk & 1;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      qraw[j][h][0] = qraw[j][h][1] = v4i{0, 0, 0, 0};
      if (blk < NBLK && qhead < p.hr) {
        const uint16_t* src = p.q + ((size_t)b * p.hr + qhead) * D + h * HALF + 32 * qks + 16 * qc;
        qraw[j][h][0] = *reinterpret_cast<const v4i*>(src);
        qraw[j][h][1] = *reinterpret_cast<const v4i*>(src + 8);
      }
    }
  }
  // head weights: result register j of block mb in this lane is head
  // 32 mb + 8 (j / 4) + 4 kh + j % 4, four consecutive heads per group
  uint2 wraw[MB][4];
  const uint16_t* wb = p.w + (size_t)b * p.hr;
  const bool w8 = (reinterpret_cast<uintptr_t>(p.w) & 7u) == 0;   // 8-byte loads when aligned
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int head0 = 32 * mb + 8 * g + 4 * kh;
      wraw[mb][g] = make_uint2(0u, 0u);
      if (head0 < p.hr) {                          // hr is a multiple of 8: all four heads are real
        if (w8) {
          wraw[mb][g] = *reinterpret_cast<const uint2*>(wb + head0);
        } else {
          wraw[mb][g] = make_uint2((uint32_t)wb[head0] | ((uint32_t)wb[head0 + 1] << 16),
                                   (uint32_t)wb[head0 + 2] | ((uint32_t)wb[head0 + 3] << 16));
        }
      }
    }

  int step_page = 0;
  if constexpr (PAGED) {
    if (lane < S) {
      const int sb = 32 * static_chunk(lane);
      step_page = p.block_table[(size_t)b * p.max_blocks + (sb >> p.page_shift)];
      step_page = min(max(step_page, 0), p.num_pages - 1);
    }
    for (int j = tid; j < npool; j += DS_NT) {
      const int sb = 32 * (nstat + j);
      const int pg = p.block_table[(size_t)b * p.max_blocks + (sb >> p.page_shift)];
      pool_page[j] = min(max(pg, 0), p.num_pages - 1);
    }
  }
  for (int i = tid; i < DS_WAVES * DS_CAP; i += DS_NT) (&step_chunk[0][0])[i] = -1;
  // the pool's first claimers are at least a few steps away: one lane of the
  // sequence's first workgroup tags the counter now, so that claims find it
  // tagged (a claimer that still finds it stale re-tags it itself)
  if (x == 0 && tid == 0 && npool > 0) {
    unsigned long long cur = atomicAdd(pool, 0ull);
    while ((uint32_t)(cur >> 32) != tag) {
      const unsigned long long seen = atomicCAS(pool, cur, (unsigned long long)tag << 32);
      if (seen == cur) break;
      cur = seen;
    }
    __builtin_amdgcn_s_waitcnt(0);
  }
  __syncthreads();   // pool pages and the step table are in place
  // Each step gets a descriptor based at its first key whose record limit
  // covers only the keys below len (of the page, when paged): the range
  // check then applies to the lane offsets alone.
  const uint8_t* rows_b = p.cache + (size_t)b * p.Lmax * D;
  const float* ks_b = p.k_scale + (size_t)b * p.Lmax;
  // loads local step `sub` of the wave, chunk c (c < 0: nothing, the loads
  // read zeros without touching memory)
  auto fetch = [&](int slot, int sub, int c) {
    c = __builtin_amdgcn_readfirstlane(c);   // uniform: keeps the descriptors in scalar registers
    const int s0 = 32 * max(c, 0);
    const uint8_t* rbase = rows_b + (size_t)s0 * D;
    const float* kbase = ks_b + s0;
    const int valid = __builtin_amdgcn_readfirstlane(c < 0 ? 0 : min(max(len - s0, 0), 32));
    if constexpr (PAGED) {
      const int pg = c < 0 ? 0 : sub < S ? __builtin_amdgcn_readlane(step_page, min(sub, 63)) : pool_page[c - nstat];
      const int off = s0 & ((1 << p.page_shift) - 1);
      rbase = p.cache + (((size_t)pg << p.page_shift) + off) * D;
      kbase = p.k_scale + ((size_t)pg << p.page_shift) + off;
    }
    const __amdgpu_buffer_rsrc_t rr = buf_rsrc(rbase, (uint32_t)valid * D);
    const __amdgpu_buffer_rsrc_t kr = buf_rsrc(kbase, (uint32_t)valid * 4u);
#pragma unroll
    for (int i = 0; i < NLD; ++i)
      raw[slot][i] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rr, 1024 * i + 16 * lane, 0, 0));
    kss[slot] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(kr, 4 * col, 0, 0));
  };
  // Local step u reads chunk cid[u % PF]: a static chunk while u < S, then
  // pool chunks, a batch of DS_PF consecutive pool entries per ring turn.
  // The batch for the steps fetched during ring turn g (steps g + PF ..
  // g + 2 PF - 1) is claimed at the start of turn g - PF and read at the
  // start of turn g: loads complete in order, so by then it has returned
  // without an extra wait.
  int cid[DS_PF];
  unsigned long long bclm;               // the batch claim in flight (lane 0)
  bool dry = npool == 0;                 // no pool entry left to claim
  auto claim = [&]() {                   // only lane 0's value is used
    if (lane == 0) bclm = atomicAdd(pool, (unsigned long long)DS_PF);
  };
  auto batch = [&](unsigned long long v) -> int {   // first pool entry of a batch, or -1 (uniform)
    int j = 0;
    if (lane == 0) j = (int)min(take(v), (uint32_t)npool);
    j = __builtin_amdgcn_readfirstlane(j);
    if (j >= npool) {
      dry = true;
      j = -1;
    }
    return j;
  };
  // chunk of local step `sub` in a turn whose batch starts at pool entry jb
  auto chunk_of = [&](int sub, int jb) -> int {
    if (sub < S) return static_chunk(sub);
    if (jb < 0 || sub >= DS_CAP) return -1;
    const int j = jb + (sub & (DS_PF - 1));
    return j < npool ? nstat + j : -1;
  };
  int jb = -1;
  if (S == 0 && !dry) {                  // the first turn is already pool: claim it now
    claim();
    jb = batch(bclm);
  }
#pragma unroll
  for (int u = 0; u < DS_PF; ++u) cid[u] = chunk_of(u, jb);
  if (DS_PF >= S && !dry) claim();       // the batch of the next turn, before the first loads
#pragma unroll
  for (int u = 0; u < DS_PF; ++u) fetch(u, u, cid[u]);

  // ---- the query's limbs.  Limb 0 is the block rounded to e4m3 on the
  // grid of its largest element, limb 1 the exact residual rounded the same
  // way (a bf16 value has 8 significant bits, a limb 4).  Staged in operand
  // order, [mb][kk][c][lane][16 bytes] with kk = limb * KS + ks, and one
  // scale word per (mb, lane): byte kk for lane (row, c).
  // (at H = 128 the limbs outgrow the transpose buffer: they take the
  // score stage, and their scales the transpose buffer)
  constexpr bool QBIG = MB * NK * 2 * 64 * 16 > (int)sizeof(ktr);
  uint8_t* lstage = QBIG ? reinterpret_cast<uint8_t*>(sc_stage) : &ktr[0][0];
  int* lscale = QBIG ? reinterpret_cast<int*>(&ktr[0][0]) : reinterpret_cast<int*>(sc_stage);
  static_assert(MB * NK * 2 * 64 * 16 <= (int)(QBIG ? sizeof(sc_stage) : sizeof(ktr)) &&
                MB * 64 * 4 <= (int)(QBIG ? sizeof(ktr) : sizeof(sc_stage)), "limb staging");
#pragma unroll
  for (int jb = 0; jb < QB; ++jb) {
    const int blk = tid + DS_NT * jb;
    if (blk >= NBLK) break;
    const int qhead = blk / (KS * 2), ks = (blk >> 1) % KS, c = blk & 1;
    const int mb = qhead >> 5, row = qhead & 31;
    float v[32];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t wd = (uint32_t)qraw[jb][h][i >> 3][(i & 7) >> 1];
        v[16 * h + i] = __uint_as_float((i & 1) ? (wd & 0xFFFF0000u) : (wd << 16));
      }
#pragma unroll
    for (int limb = 0; limb < 2; ++limb) {
      float m = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) m = fmaxf(m, fabsf(v[i]));
      const bool keep = m >= LIMB_MIN;
      const int e = keep ? limb_exp(m) : 0;
      const float down = keep ? __uint_as_float((uint32_t)(127 - e) << 23) : 0.f;   // 2^-e; 0 drops the block
      const float up = __uint_as_float((uint32_t)(127 + e) << 23);                   // 2^e
      const int kk = limb * KS + ks;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t w4[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int i = 16 * h + 4 * g;
          // the matrix cores' own e4m3 conversion (round to nearest even,
          // subnormals kept), then the exact residual of that rounding
          int pk = __builtin_amdgcn_cvt_pk_fp8_f32(v[i] * down, v[i + 1] * down, 0, false);
          pk = __builtin_amdgcn_cvt_pk_fp8_f32(v[i + 2] * down, v[i + 3] * down, pk, true);
          w4[g] = (uint32_t)pk;
          v[i] = fmaf(-__builtin_amdgcn_cvt_f32_fp8(pk, 0), up, v[i]);
          v[i + 1] = fmaf(-__builtin_amdgcn_cvt_f32_fp8(pk, 1), up, v[i + 1]);
          v[i + 2] = fmaf(-__builtin_amdgcn_cvt_f32_fp8(pk, 2), up, v[i + 2]);
          v[i + 3] = fmaf(-__builtin_amdgcn_cvt_f32_fp8(pk, 3), up, v[i + 3]);
        }
        *reinterpret_cast<v4i*>(lstage + (((mb * NK + kk) * 2 + c) * 64 + row + 32 * h) * 16) =
            v4i{(int)w4[0], (int)w4[1], (int)w4[2], (int)w4[3]};
      }
      // lane (row, c) holds the scales of blocks (ks, c) of both limbs
      reinterpret_cast<uint8_t*>(&lscale[mb * 64 + row + 32 * c])[kk] = (uint8_t)(e + 127);
    }
  }
  for (int i = tid; i < HBINS; i += DS_NT) hist[i] = 0u;
  __syncthreads();
  v8i qa[MB][NK];
  int qsc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    qsc[mb] = lscale[mb * 64 + lane];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const v4i lo = *reinterpret_cast<const v4i*>(lstage + (((mb * NK + kk) * 2 + 0) * 64 + lane) * 16);
      const v4i hi = *reinterpret_cast<const v4i*>(lstage + (((mb * NK + kk) * 2 + 1) * 64 + lane) * 16);
      qa[mb][kk] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  }
  float wr[MB][16];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t wd = (j & 2) ? wraw[mb][j >> 2].y : wraw[mb][j >> 2].x;
      wr[mb][j] = __uint_as_float((j & 1) ? (wd & 0xFFFF0000u) : (wd << 16));
    }
  __syncthreads();   // every lane has its operands before scores overwrite the stage

  uint8_t* tr = ktr[wave];
  // this lane's operand chunks: key `col`, chunks kh*NLD + i of its row
  const int rswz = (col / RPB) % CPR;
  // the ring is unrolled inside a rolled loop; with unconditional loads every
  // slot keeps its registers across iterations
  int nproc = 0;                         // steps read so far (they are the first nproc)
#pragma unroll 1
  for (int g = 0; g < DS_CAP && cid[0] >= 0; g += DS_PF) {
    // the batch of the steps this turn fetches, and the claim for the next turn's
    int jn = -1;
    if (g + DS_PF >= S && g + DS_PF < DS_CAP && !dry) jn = batch(bclm);
    if (g + 2 * DS_PF >= S && g + 2 * DS_PF < DS_CAP && !dry) claim();
#pragma unroll
    for (int u = 0; u < DS_PF; ++u) {
      const int sub = g + u;
      const int ccur = cid[u];
      const int s0 = 32 * ccur;
      // through the wave's LDS transpose into per-key operand order
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const int byte = 1024 * i + 16 * lane;
        const int r = byte / D, c = (byte % D) / 16;
        *reinterpret_cast<v4i*>(tr + r * D + 16 * (c ^ ((r / RPB) % CPR))) = raw[u][i];
      }
      if (kh == 0) kst[wave][col] = kss[u];
      const int nxt = sub + DS_PF;
      const int cn = chunk_of(nxt, jn);
      cid[u] = cn;
      fetch(u, nxt, cn);
      if (lane == 0 && ccur >= 0) step_chunk[wave][sub] = ccur;
      if (ccur >= 0) nproc = sub + 1;
      wave_lds_sync();
      v4i cur[NLD];
#pragma unroll
      for (int i = 0; i < NLD; ++i)
        cur[i] = *reinterpret_cast<const v4i*>(tr + col * D + 16 * ((kh * NLD + i) ^ rswz));
      const float cks = kst[wave][col];
      wave_lds_sync();   // every lane has read before the next step overwrites

      v16f acc[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[mb] = v16f{};
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const int ks = kk % KS;
        const v8i bop = v8i{cur[2 * ks][0], cur[2 * ks][1], cur[2 * ks][2], cur[2 * ks][3],
                            cur[2 * ks + 1][0], cur[2 * ks + 1][1], cur[2 * ks + 1][2], cur[2 * ks + 1][3]};
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          if (kk == 0) acc[mb] = mfma_kk<0>(qa[mb][kk], bop, acc[mb], qsc[mb]);
          else if (kk == 1) acc[mb] = mfma_kk<1>(qa[mb][kk], bop, acc[mb], qsc[mb]);
          else if (kk == 2) acc[mb] = mfma_kk<2>(qa[mb][kk], bop, acc[mb], qsc[mb]);
          else acc[mb] = mfma_kk<3>(qa[mb][kk], bop, acc[mb], qsc[mb]);
        }
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
      if (kh == 0 && ccur >= 0 && s < len) {
        // NaN ranks lowest (a bit test: the library builds with -fno-honor-nans)
        const uint32_t key = (__float_as_uint(score) & 0x7FFFFFFFu) > 0x7F800000u ? 0u : ordered_key(score);
        reinterpret_cast<uint32_t*>(sc_stage)[sub * (32 * DS_WAVES) + wave * 32 + col] = key;
        atomicAdd(&hist[key >> 20], 1u);
      }
    }
  }
  if (lane == 0) wave_steps[wave] = nproc;
  __syncthreads();

  // ---- tail.  Thread t holds fine bins 16t .. 16t + 15 (thread order = bin
  // order), which are exactly coarse bin t.  The workgroup's histograms go
  // out packed: words [0, HBINS/2) hold the fine bins in pairs, [HBINS/2, PW)
  // the coarse bins in pairs.
  static_assert(FPC == 16 && CBINS == DS_NT, "one coarse bin per thread");
  uint32_t* gh = p.hist + ((size_t)b * nwg + x) * PW;
  uint32_t h16[16], mine = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const v4i t = reinterpret_cast<const v4i*>(hist)[4 * tid + q];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      h16[4 * q + j] = (uint32_t)t[j];
      mine += (uint32_t)t[j];
    }
  }
  const uint32_t next_coarse = (uint32_t)__shfl_down((int)mine, 1);
  if ((tid & 1) == 0) gh[HBINS / 2 + tid / 2] = mine | (next_coarse << 16);
  // Its min(k, n) best keys and the rest of their boundary bin: a suffix sum
  // gives every bin the number of keys in higher bins, which becomes the
  // bin's first output position.
  const int incl = wave_incl_sum((int)mine);
  int* wsum = reinterpret_cast<int*>(ktr);     // the transpose area is free now
  if (lane == 63) wsum[wave] = incl;
  if (tid == 0) {                              // a workgroup whose steps all went to others keeps nothing
    sh_cut[0] = HBINS;
    sh_cut[1] = 0;
  }
  __syncthreads();
  int higher_waves = 0, total = 0;
#pragma unroll
  for (int w2 = 0; w2 < DS_WAVES; ++w2) {
    const int v2 = wsum[w2];
    total += v2;
    higher_waves += w2 > wave ? v2 : 0;
  }
  const int wave_tot = __builtin_amdgcn_readlane(incl, 63);
  uint32_t above = (uint32_t)(higher_waves + wave_tot - incl);   // keys in bins above this thread's
  const uint32_t kk_w = (uint32_t)min(p.topk, total);
  uint32_t first[16];
#pragma unroll
  for (int j = 15; j >= 0; --j) {
    if (above < kk_w && above + h16[j] >= kk_w) {
      sh_cut[0] = 16 * tid + j;
      sh_cut[1] = (int)(above + h16[j]);   // keys at or above the boundary bin
    }
    first[j] = above;                       // output position of the bin's first key
    above += h16[j];
  }
#pragma unroll
  for (int q = 0; q < 4; ++q)
    reinterpret_cast<v4i*>(hist)[4 * tid + q] =
        v4i{(int)first[4 * q], (int)first[4 * q + 1], (int)first[4 * q + 2], (int)first[4 * q + 3]};
  __syncthreads();
  const uint32_t dcut = (uint32_t)sh_cut[0];
  // the fine bins go out only from the coarse bin of the cut up: the select
  // never needs a list's fine counts below its cut (the bin of the
  // sequence's k-th score is at or above every list's cut), and masks them
#pragma unroll
  for (int q = 0; q < 2; ++q)
    if (16u * tid + 15u >= dcut)
      reinterpret_cast<v4i*>(gh)[2 * tid + q] =
          v4i{(int)(h16[8 * q] | (h16[8 * q + 1] << 16)), (int)(h16[8 * q + 2] | (h16[8 * q + 3] << 16)),
              (int)(h16[8 * q + 4] | (h16[8 * q + 5] << 16)), (int)(h16[8 * q + 6] | (h16[8 * q + 7] << 16))};
  // the workgroup's list: positions below DS_KCAP (positions count kept keys)
  const __amdgpu_buffer_rsrc_t crs = buf_rsrc(p.cand + ((size_t)b * nwg + x) * DS_KCAP, DS_KCAP * 8u);
  uint32_t* dummy = reinterpret_cast<uint32_t*>(ktr) + 64;   // per thread, past wsum
  int nslot = 0;                         // stage slots in use: the longest wave's steps
#pragma unroll
  for (int w2 = 0; w2 < DS_WAVES; ++w2) nslot = max(nslot, wave_steps[w2]);
  nslot *= 32 * DS_WAVES;
  // Eight slots per thread per pass, as two runs of four consecutive slots.
  // Stage slot e is key e % 32 of step e / 128 of wave (e / 32) % 4, so a run
  // lies in one 32-key step: one chunk lookup and one 16-byte read per run.
  // nslot is a multiple of 128 and at most DS_KCAP, a whole number of
  // passes, so every read stays in the stage; runs past nslot are masked.
  constexpr int SCAT = 8;
  static_assert(DS_KCAP % (SCAT * DS_NT) == 0, "whole passes over the stage");
  const uint32_t* stage = reinterpret_cast<const uint32_t*>(sc_stage);
  for (int e0 = 0; e0 < nslot; e0 += SCAT * DS_NT) {
    uint32_t key[SCAT];
    int sidx[SCAT];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int e = e0 + h * (4 * DS_NT) + 4 * tid;
      const v4i kv = *reinterpret_cast<const v4i*>(stage + e);
      const int cr = step_chunk[(e >> 5) % DS_WAVES][e / (32 * DS_WAVES)];
      const int c = e < nslot ? cr : -1;
      const int s = 32 * c + (e & 31);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        key[4 * h + j] = (uint32_t)kv[j];
        sidx[4 * h + j] = (c >= 0 && s + j < len) ? s + j : -1;
      }
    }
    // Without branches: a key that is not kept adds 0 to this thread's own
    // dummy word, and its store goes to the first byte past the list's
    // record limit, where the buffer store writes nothing.
    uint32_t pos[SCAT];
#pragma unroll
    for (int u = 0; u < SCAT; ++u) {
      const bool kept = sidx[u] >= 0 && (key[u] >> 20) >= dcut;
      pos[u] = atomicAdd(kept ? &hist[key[u] >> 20] : &dummy[tid], kept ? 1u : 0u);
      pos[u] = kept ? pos[u] * 8u : DS_KCAP * 8u;
    }
#pragma unroll
    for (int u = 0; u < SCAT; ++u)
      __builtin_amdgcn_raw_buffer_store_b64(v2u{key[u], (uint32_t)sidx[u]}, crs, (int)pos[u], 0, 0);
  }
  if (tid == 0) p.wgcut[(size_t)b * nwg + x] = make_int2(sh_cut[0], sh_cut[1]);
}

// ---------------------------------------------------------------------------
// select: one workgroup per sequence over its workgroups' lists
// ---------------------------------------------------------------------------

namespace {

struct SelShared {
  uint32_t chist[CBINS];              // the sequence's coarse histogram
  uint32_t fhist[FPC];                // its fine bins inside the boundary coarse bin
  uint32_t rhist[SL_NT];              // radix bins of the boundary-bin resolution
  uint32_t fw[DS_MAXWG][FPC];         // per list: those fine bins
  __attribute__((aligned(16))) int wtot[SL_NT / 64];
  int2 cut[DS_MAXWG];                 // per list: (lowest bin kept, entries)
  int gt[DS_MAXWG];                   // per list: entries above the boundary bin
  int base[DS_MAXWG + 1];             // list offsets in the concatenation of the prefixes read
  int bc[4];
  int ntie;
};

// exclusive scan of v over the workgroup; *total gets the sum
__device__ int sl_scan(int v, SelShared& sh, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int incl = wave_incl_sum(v);
  if (lane == 63) sh.wtot[wave] = incl;
  __syncthreads();
  int pre = 0, tot = 0;
  static_assert(SL_NT % 256 == 0, "wave totals in 16-byte groups");
#pragma unroll
  for (int g = 0; g < SL_NT / 256; ++g) {
    const v4i x4 = reinterpret_cast<const v4i*>(sh.wtot)[g];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      pre += (4 * g + j < wave) ? x4[j] : 0;
      tot += x4[j];
    }
  }
  __syncthreads();
  *total = tot;
  return pre + incl - v;
}

}  // namespace

__global__ void __launch_bounds__(SL_NT) decode_select_kernel(DecodeParams p, int nwg) {
  extern __shared__ __attribute__((aligned(16))) uint32_t dyn[];
  __shared__ SelShared sh;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int k = p.topk;
  int* out = p.out_idx + (size_t)b * k;
  float* osc = p.out_score ? p.out_score + (size_t)b * k : nullptr;
  const uint2* lists = p.cand + (size_t)b * nwg * DS_KCAP;
  const uint32_t* ph = p.hist + (size_t)b * nwg * PW;
  if (tid == 0) p.hdr[b].gen += 1u;   // the next call's pool tag differs from this one's

  // A. one round of loads: the length, the lists' cuts and coarse histogram
  //    words (words of lists past the active ones are read but not used)
  const int n = seq_len(p, b);
  const int2 cutv = tid < nwg ? p.wgcut[(size_t)b * nwg + tid] : make_int2(0, 0);
  constexpr int CW = DS_MAXWG * (CBINS / 2) / SL_NT;
  uint32_t cw[CW];
#pragma unroll
  for (int j = 0; j < CW; ++j) {
    const int i = tid + SL_NT * j;
    cw[j] = i < nwg * (CBINS / 2) ? ph[(size_t)(i / (CBINS / 2)) * PW + HBINS / 2 + i % (CBINS / 2)] : 0u;
  }
  const int nchunk = (n + 31) >> 5;
  const int nact = min(nwg, (nchunk + DS_WAVES - 1) / DS_WAVES);
  const int nw = (n + 31) >> 5;
  const int nw4 = (nw + 3) & ~3;       // bitmap words, rounded up to whole 16-byte groups (kept zero)
  uint32_t* bm = dyn;                  // selected keys
  uint32_t* tb = dyn + nw4;            // keys tied with the k-th, later word prefix counts
  int* obuf = reinterpret_cast<int*>(dyn + 2 * nw4);        // the output row, staged
  float* osbuf = reinterpret_cast<float*>(dyn + 2 * nw4 + k);
  for (int i = tid; i < nw4; i += SL_NT) {
    bm[i] = 0u;
    tb[i] = 0u;
  }
  if (tid < nact) {
    sh.cut[tid] = cutv;
    sh.gt[tid] = 0;
  }
  if (tid < CBINS) sh.chist[tid] = 0u;
  if (tid < FPC) sh.fhist[tid] = 0u;
  if (tid == 0) sh.ntie = 0;
  // the list holding entry i of the concatenation: the last w with base[w] <= i
  auto list_of = [&](int i) {
    int lo = 0;
#pragma unroll
    for (int st = DS_MAXWG / 2; st >= 1; st >>= 1)
      if (lo + st < nact && sh.base[lo + st] <= i) lo += st;
    return lo;
  };
  // base[] over per-list counts cnt (lanes w < nact of wave 0)
  auto set_bases = [&](int cnt) {
    if (tid < 64) {
      const int v = tid < nact ? cnt : 0;
      const int incl = wave_incl_sum(v);
      if (tid < nact) sh.base[tid] = incl - v;
      if (tid == 63) sh.base[nact] = incl;
    }
  };

  if (n <= k) {                       // every key is kept: position = index
    set_bases(tid < nact ? cutv.y : 0);
    __syncthreads();
    for (int i = tid; i < sh.base[nact]; i += SL_NT) {
      const int w = list_of(i);
      const uint2 c = lists[(size_t)w * DS_KCAP + (i - sh.base[w])];
      out[c.y] = (int)c.y;
      if (osc) osc[c.y] = key_to_float(c.x);
    }
    for (int j = n + tid; j < k; j += SL_NT) {
      out[j] = -1;
      if (osc) osc[j] = -__builtin_inff();
    }
    return;
  }
  __syncthreads();

  // B. the sequence's coarse histogram and the coarse bin c* of the k-th score
#pragma unroll
  for (int j = 0; j < CW; ++j) {
    const int i = tid + SL_NT * j;
    if (i < nact * (CBINS / 2)) {
      const int c2 = i % (CBINS / 2);
      if (cw[j] & 0xFFFFu) atomicAdd(&sh.chist[2 * c2], cw[j] & 0xFFFFu);
      if (cw[j] >> 16) atomicAdd(&sh.chist[2 * c2 + 1], cw[j] >> 16);
    }
  }
  __syncthreads();
  {
    // bins in descending order: thread t holds bin 255 - t
    const int hv = tid < CBINS ? (int)sh.chist[CBINS - 1 - tid] : 0;
    int tot;
    const int ab = sl_scan(hv, sh, &tot);   // keys in higher coarse bins
    if (tid < CBINS && ab < k && ab + hv >= k) {
      sh.bc[0] = CBINS - 1 - tid;
      sh.bc[1] = ab;
    }
    __syncthreads();
  }
  const int cstar = sh.bc[0];
  // C. per list: its keys in the coarse bins above c* (gt) and its fine bins
  //    inside c* (fw), summed over the lists into fhist; loads first
  constexpr int CI = (DS_MAXWG * (CBINS / 2 + FPC / 2) + SL_NT - 1) / SL_NT;
  uint32_t cv[CI];
#pragma unroll
  for (int j = 0; j < CI; ++j) {
    const int i = tid + SL_NT * j;
    size_t addr = 0;
    if (i < nact * (CBINS / 2)) {
      addr = (size_t)(i / (CBINS / 2)) * PW + HBINS / 2 + i % (CBINS / 2);
    } else {
      const int i2 = i - nact * (CBINS / 2);
      addr = (size_t)(i2 / (FPC / 2)) * PW + (FPC / 2) * cstar + i2 % (FPC / 2);
    }
    cv[j] = i < nact * (CBINS / 2 + FPC / 2) ? ph[addr] : 0u;
  }
#pragma unroll
  for (int j = 0; j < CI; ++j) {
    const int i = tid + SL_NT * j;
    const uint32_t t = cv[j];
    if (i < nact * (CBINS / 2)) {
      const int w = i / (CBINS / 2), c2 = i % (CBINS / 2);
      const int cnt = (2 * c2 > cstar ? (int)(t & 0xFFFFu) : 0) + (2 * c2 + 1 > cstar ? (int)(t >> 16) : 0);
      if (cnt) atomicAdd(&sh.gt[w], cnt);
    } else if (i < nact * (CBINS / 2 + FPC / 2)) {
      const int i2 = i - nact * (CBINS / 2);
      const int w = i2 / (FPC / 2), jj = i2 % (FPC / 2);
      // fine bins below the list's cut were not written (stale words): zero
      const int lo = sh.cut[w].x - FPC * cstar;
      const uint32_t f0 = 2 * jj >= lo ? (t & 0xFFFFu) : 0u, f1 = 2 * jj + 1 >= lo ? (t >> 16) : 0u;
      sh.fw[w][2 * jj] = f0;
      sh.fw[w][2 * jj + 1] = f1;
      if (f0) atomicAdd(&sh.fhist[2 * jj], f0);
      if (f1) atomicAdd(&sh.fhist[2 * jj + 1], f1);
    }
  }
  __syncthreads();
  if (tid < 64) {
    const int lane = tid;
    const int h = lane < FPC ? (int)sh.fhist[lane] : 0;
    int incl = h;                     // keys in fine bins lane.. of the coarse bin
#pragma unroll
    for (int o = 1; o < FPC; o <<= 1) {
      const int t = __shfl_down(incl, o);
      if (lane + o < FPC) incl += t;
    }
    const int ab2 = sh.bc[1] + incl - h;
    if (lane < FPC && ab2 < k && ab2 + h >= k) {
      sh.bc[2] = lane;                 // fine bin of the k-th score within the coarse bin
      sh.bc[3] = ab2;                  // keys above it
    }
  }
  __syncthreads();
  const int jstar = sh.bc[2];
  const uint32_t dstar = (uint32_t)(FPC * cstar + jstar);
  const int need = k - sh.bc[3];       // keys still to take from bin d* (>= 1)
  {
    int gt = 0, pref = 0;
    if (tid < nact) {
      gt = sh.gt[tid];
#pragma unroll
      for (int j = 0; j < FPC; ++j) gt += j > jstar ? (int)sh.fw[tid][j] : 0;
      pref = gt + (int)sh.fw[tid][jstar];
    }
    __syncthreads();                   // every gt read before it is rewritten
    if (tid < nact) sh.gt[tid] = gt;
    set_bases(pref);
  }
  __syncthreads();
  const int total = sh.base[nact];

  // D. the candidates: entry i of the concatenation is entry i - base[w] of
  //    list w; the first gt_w of each list lie above bin d* and are selected
  //    outright.  Entries tid + SL_NT j, j < SL_REG, are held in registers
  //    (5120: at k = 2048 the prefixes hold k plus the d* bin, up to about
  //    4200 entries); more (a larger k, or many equal scores) are read again
  //    from the lists at every pass over the candidates.
  constexpr int SL_REG = 5;
  uint2 rc[SL_REG];
  bool ra[SL_REG];
#pragma unroll
  for (int j = 0; j < SL_REG; ++j) {
    const int i = tid + SL_NT * j;
    rc[j] = make_uint2(0u, 0u);
    ra[j] = false;
    if (i < total) {
      const int w = list_of(i);
      const int e = i - sh.base[w];
      rc[j] = lists[(size_t)w * DS_KCAP + e];
      ra[j] = e < sh.gt[w];
    }
  }
  // calls body(key, index, above) for every candidate
  auto for_all = [&](auto body) {
#pragma unroll
    for (int j = 0; j < SL_REG; ++j)
      if (tid + SL_NT * j < total) body(rc[j].x, (int)rc[j].y, ra[j]);
    for (int i = tid + SL_NT * SL_REG; i < total; i += SL_NT) {
      const int w = list_of(i);
      const int e = i - sh.base[w];
      const uint2 c = lists[(size_t)w * DS_KCAP + e];
      body(c.x, (int)c.y, e < sh.gt[w]);
    }
  };
  for_all([&](uint32_t, int s, bool above) {
    if (above) atomicOr(&bm[s >> 5], 1u << (s & 31));
  });
  // calls body(key, index) for every candidate of bin d*
  auto for_boundary = [&](auto body) {
    for_all([&](uint32_t key, int s, bool above) {
      if (!above) body(key, s);
    });
  };
  // E. exact k-th key among them (they share the top 12 bits): two rounds of
  //    1024 bins, one per thread
  int need2 = need;
  uint32_t prefix = dstar << 20;
  uint32_t pmask = 0xFFF00000u;
  static_assert(SL_NT == 1024, "one radix bin per thread");
#pragma unroll 1
  for (int shift = 10; shift >= 0; shift -= 10) {
    sh.rhist[tid] = 0u;
    __syncthreads();
    for_boundary([&](uint32_t key, int) {
      if ((key & pmask) == prefix) atomicAdd(&sh.rhist[(key >> shift) & 1023u], 1u);
    });
    __syncthreads();
    // bins in descending order: thread t holds bin 1023 - t
    const int hv = (int)sh.rhist[SL_NT - 1 - tid];
    int t2;
    const int ab = sl_scan(hv, sh, &t2);   // entries in higher bins
    if (ab < need2 && ab + hv >= need2) {
      sh.bc[2] = SL_NT - 1 - tid;
      sh.bc[3] = ab;
    }
    __syncthreads();
    prefix |= (uint32_t)sh.bc[2] << shift;
    pmask |= 1023u << shift;
    need2 -= sh.bc[3];
  }
  const uint32_t kstar = prefix;       // the k-th key; need2 of its ties are kept
  for_boundary([&](uint32_t key, int s) {
    if (key > kstar) {
      atomicOr(&bm[s >> 5], 1u << (s & 31));
    } else if (key == kstar) {
      atomicOr(&tb[s >> 5], 1u << (s & 31));
      atomicAdd(&sh.ntie, 1);
    }
  });
  __syncthreads();

  // F. ties with the k-th key: when more than need2 keys tie, the need2
  //    lowest indices (otherwise every tied key is taken)
  const int wpt = (nw + SL_NT - 1) / SL_NT;   // bitmap words per thread, contiguous
  // uniform: at most four words per thread, as one 16-byte group (thread t
  // holds words 4t .. 4t + 3, those past nw are zero)
  const bool w4 = nw4 <= 4 * SL_NT;
  const bool g4 = 4 * tid < nw4;       // this thread's group exists
  if (sh.ntie == need2 && w4) {
    if (g4) reinterpret_cast<v4i*>(bm)[tid] |= reinterpret_cast<const v4i*>(tb)[tid];
  } else if (sh.ntie == need2) {      // uniform
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
      uint32_t xw = tb[wd];
      while (xw) {
        const int bpos = __ffs(xw) - 1;
        xw &= xw - 1;
        if (before < need2) bm[wd] |= 1u << bpos;
        ++before;
      }
    }
  }
  __syncthreads();

  // G. ascending output: the rank of a selected key is the number of
  //    selected keys below it (word prefix counts in tb, then a popcount)
  if (w4) {
    const v4i b4 = g4 ? reinterpret_cast<const v4i*>(bm)[tid] : v4i{0, 0, 0, 0};
    const int c0 = __popc(b4[0]), c1 = __popc(b4[1]), c2 = __popc(b4[2]), c3 = __popc(b4[3]);
    int t4;
    const int pos = sl_scan(c0 + c1 + c2 + c3, sh, &t4);
    if (!osc) {                        // uniform: indices straight from the bitmap
      int q = pos;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t xw = (uint32_t)b4[i];
        while (xw) {
          const int bpos = __ffs(xw) - 1;
          xw &= xw - 1;
          if (q < k) out[q] = 32 * (4 * tid + i) + bpos;
          ++q;
        }
      }
      return;                          // exactly k bits are set: every position is written
    }
    if (g4) reinterpret_cast<v4i*>(tb)[tid] = v4i{pos, pos + c0, pos + c0 + c1, pos + c0 + c1 + c2};
  } else {
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
      tb[wd] = (uint32_t)pos;
      pos += __popc(bm[wd]);
    }
  }
  __syncthreads();
  for_all([&](uint32_t key, int s, bool) {
    const uint32_t wbits = bm[s >> 5];
    if ((wbits >> (s & 31)) & 1u) {
      const int pos = (int)tb[s >> 5] + __popc(wbits & ((1u << (s & 31)) - 1u));
      if (pos < k) {
        obuf[pos] = s;
        osbuf[pos] = key_to_float(key);
      }
    }
  });
  __syncthreads();
  // exactly k keys are selected: every position is written
  for (int j = tid; j < k; j += SL_NT) {
    out[j] = obuf[j];
    if (osc) osc[j] = osbuf[j];
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

static int score_workgroups(int Lmax) { return (Lmax + DS_KPB - 1) / DS_KPB; }

size_t decode_select_lds_bytes(int Lmax, int topk) {
  const size_t nw = (((size_t)Lmax + 31) / 32 + 3) & ~(size_t)3;   // bitmap words in whole 16-byte groups
  return (2 * nw + 2 * (size_t)topk) * sizeof(uint32_t);
}

bool decode_supported(int H, int D, int Lmax) {
  if (!decode_head_width(H)) return false;
  if (D != 64 && D != 128) return false;
  if (score_workgroups(Lmax) > DS_MAXWG) return false;
  return decode_select_lds_bytes(Lmax, MAX_TOPK) + sizeof(SelShared) <= 160 * 1024;
}

DecodeWsSizes decode_ws_sizes(int Lmax) {
  DecodeWsSizes z;
  z.nwg = (size_t)score_workgroups(Lmax);
  z.hist_words = z.nwg * PW;
  z.cand_entries = z.nwg * DS_KCAP;
  return z;
}

template <int H, int D>
static void launch_score(const DecodeParams& p, hipStream_t stream) {
  static_assert(H <= 128, "head width");
  dim3 grid(score_workgroups(p.Lmax) * p.B);
  if (p.block_table) hipLaunchKernelGGL((decode_score_kernel<H, D, true>), grid, dim3(DS_NT), 0, stream, p);
  else hipLaunchKernelGGL((decode_score_kernel<H, D, false>), grid, dim3(DS_NT), 0, stream, p);
}

hipError_t decode_launch(const DecodeParams& p, int H, int D, hipStream_t stream) {
  H = decode_head_width(H);
  if (H == 128 && D == 128) launch_score<128, 128>(p, stream);
  else if (H == 128 && D == 64) launch_score<128, 64>(p, stream);
  else if (H == 64 && D == 128) launch_score<64, 128>(p, stream);
  else if (H == 64 && D == 64) launch_score<64, 64>(p, stream);
  else if (H == 32 && D == 128) launch_score<32, 128>(p, stream);
  else if (H == 32 && D == 64) launch_score<32, 64>(p, stream);
  else if (H == 16 && D == 128) launch_score<16, 128>(p, stream);
  else if (H == 16 && D == 64) launch_score<16, 64>(p, stream);
  else return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = decode_select_lds_bytes(p.Lmax, p.topk);
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(decode_select_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_select_kernel, dim3(p.B), dim3(SL_NT), lds, stream, p, score_workgroups(p.Lmax));
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// scratch of the allocation-free decode entry point
// ---------------------------------------------------------------------------

// One copy per device, held from the library's load to the end of the
// process; every allocation-free call on a device shares it.
constexpr size_t DECODE_SCRATCH_BYTES = size_t(48) << 20;
static __device__ __align__(256) uint8_t scratch[DECODE_SCRATCH_BYTES];

size_t decode_scratch_bytes() { return DECODE_SCRATCH_BYTES; }

// Device address of the current device's copy.  In host code `scratch`
// names a host-side stand-in, so the address is looked up with
// hipGetSymbolAddress on a device's first call (that device current) and
// kept per device.
hipError_t decode_scratch(void** ptr) {
  constexpr int MAX_DEVICES = 64;
  static std::mutex mu;
  static void* addr[MAX_DEVICES] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!a) return hipErrorInvalidSymbol;
    addr[dev] = a;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace dsa
