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
// Four launches:
// 1. decode_prepare_kernel clears the per-sequence histograms and counters.
// 2. decode_score_kernel streams the fp8 cache once.  A wave reads 32 whole
//    consecutive keys per step with 16-byte loads and keeps four steps in
//    flight.  Each lane owns one key column and the D/2 contiguous bytes of
//    its half of that key; fp8 is widened to bf16 exactly (e4m3 is a subset of
//    bf16) and the contraction runs on v_mfma_f32_32x32x16_bf16 with the heads
//    on the MFMA row dimension (q stays in registers).  The per-token fp32
//    scale multiplies the fp32 score (folding it into the bf16 operand would
//    not be exact).  Scores go to a workspace row, and a 4096-bin histogram of
//    the top 12 bits of their order-preserving keys is accumulated per
//    sequence.
// 3. decode_classify_kernel (many workgroups per sequence) finds the bin of
//    the k-th score from the histogram, lists every key of a higher bin as
//    selected, and every key of that bin as a candidate.
// 4. decode_finalize_kernel (one workgroup per sequence) picks the remaining
//    keys among the candidates (radix select, ties to the lower index) and
//    writes the selection in ascending key order through an LDS bitmap.
#include "device_common.hpp"
#include "kernels.hpp"

namespace dsa {

namespace {

constexpr int DS_NT = 256;          // score kernel threads
constexpr int DS_NSUB = 64;         // 32-key steps per wave
constexpr int DS_PF = 4;            // steps in flight per wave
constexpr int DS_KPB = (DS_NT / 64) * DS_NSUB * 32;   // keys per workgroup
constexpr int HBINS = 4096;
constexpr int CL_NT = 256;          // classify threads
constexpr int CL_PER_THREAD = 32;   // scores per classify thread (8 x float4)
constexpr int CL_CHUNK = CL_NT * CL_PER_THREAD;
constexpr int FN_NT = 1024;         // finalize threads
constexpr int FN_CAP = 8192;        // candidates held in LDS by the finalize kernel

// two e4m3 (bytes 2*HI, 2*HI+1 of src) -> two bf16, exact
template <bool HI>
__device__ __forceinline__ uint32_t cvt2(uint32_t src) {
  auto r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(src, 1.0f, HI);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ int seq_len(const DecodeParams& p, int b) {
  return min(max(p.lens[b], 0), p.Lmax);   // lengths outside [0, Lmax] are clamped
}

// Bin of the k-th score: sum the histogram from the top.  Every thread of the
// block ends with (d*, count above d*) in bc[0..1].  NT threads, HBINS/NT bins each.
template <int NT>
__device__ void kth_bin(const uint32_t* gh, int k, int* wtot, int* bc) {
  constexpr int PER = HBINS / NT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t h[PER];
  int s = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    h[i] = gh[PER * tid + i];
    s += (int)h[i];
  }
  // exclusive suffix sum over threads (sum of bins above this thread's bins)
  int incl = s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_down(incl, o);
    if (lane + o < 64) incl += t;
  }
  if (lane == 0) wtot[wave] = incl;
  __syncthreads();
  int above = incl - s;
  for (int w = wave + 1; w < NT / 64; ++w) above += wtot[w];
#pragma unroll
  for (int i = PER - 1; i >= 0; --i) {
    if (above < k && above + (int)h[i] >= k) {
      bc[0] = PER * tid + i;
      bc[1] = above;
    }
    above += (int)h[i];
  }
  __syncthreads();
}

}  // namespace

template <int H, int D>
__global__ void __launch_bounds__(DS_NT, 2) decode_score_kernel(DecodeParams p) {
  constexpr int MB = (H + 31) / 32;
  constexpr int KS = D / 16;              // bf16 MFMA steps along D
  constexpr int HALF = D / 2;             // fp8 bytes of one key half
  constexpr int NLD = HALF / 16;          // 16-byte loads per lane per key
  __shared__ uint32_t hist[HBINS];
  // scores of the workgroup's keys; written out with 16-byte stores after the
  // loop so that no global store is in flight next to the MFMAs and loads
  __shared__ __attribute__((aligned(16))) float sc_stage[DS_KPB];

  const int b = blockIdx.y;
  const int len = seq_len(p, b);
  const int kbase = blockIdx.x * DS_KPB;
  if (kbase >= len) return;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int kh = lane >> 5;
  const int col = lane & 31;

  const uint8_t* cache_b = p.cache + (size_t)b * p.Lmax * D;
  const float* ks_b = p.k_scale + (size_t)b * p.Lmax;
  float* sc_b = p.scores + (size_t)b * p.ld;
  const int wbase = kbase + wave * DS_NSUB * 32;

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
  // cache prefetch ring: step u lives in slot u % DS_PF.  Loads are
  // unconditional: a key past the end of the sequence reads the last key
  // instead (its score is never stored), so no branch merges values into the
  // ring registers and no wait is forced on a load still in flight.
  v4i raw[DS_PF][NLD];
  float kss[DS_PF];
  auto fetch = [&](int slot, int s0) {
    const int s = min(s0 + col, len - 1);
#pragma unroll
    for (int i = 0; i < NLD; ++i)
      raw[slot][i] = *reinterpret_cast<const v4i*>(cache_b + (size_t)s * D + kh * HALF + 16 * i);
    kss[slot] = ks_b[s];
  };
#pragma unroll
  for (int u = 0; u < DS_PF; ++u) fetch(u, wbase + 32 * u);

  for (int i = tid; i < HBINS; i += DS_NT) hist[i] = 0u;
  __syncthreads();

  // the ring is unrolled inside a rolled loop; with unconditional loads every
  // slot keeps its registers across iterations
#pragma unroll 1
  for (int g = 0; g < DS_NSUB; g += DS_PF) {
#pragma unroll
    for (int u = 0; u < DS_PF; ++u) {
      const int sub = g + u;
      const int s0 = wbase + 32 * sub;
      {
        v4i cur[NLD];
#pragma unroll
        for (int i = 0; i < NLD; ++i) cur[i] = raw[u][i];
        const float cks = kss[u];
        fetch(u, min(s0 + 32 * DS_PF, wbase + 32 * (DS_NSUB - 1)));   // past the end: harmless reload

        // widen 16 fp8 of a load into two 8-element bf16 operands
        v8bf bop[KS];
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const uint32_t d0 = (uint32_t)cur[i][2 * h2];
            const uint32_t d1 = (uint32_t)cur[i][2 * h2 + 1];
            v4i o = v4i{(int)cvt2<false>(d0), (int)cvt2<true>(d0), (int)cvt2<false>(d1), (int)cvt2<true>(d1)};
            bop[2 * i + h2] = __builtin_bit_cast(v8bf, o);
          }
        }
        v16f acc[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[mb] = v16f{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) acc[mb] = mfma_bf16(qa[mb][ks], bop[ks], acc[mb]);
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
          sc_stage[s - kbase] = score;
          atomicAdd(&hist[ordered_key(score) >> 20], 1u);
        }
      }
    }
  }
  __syncthreads();
  // score rows are 64-float aligned (ld), kbase is a multiple of 64
  const int nval = min(DS_KPB, len - kbase);
  for (int i = tid; 4 * i < nval; i += DS_NT) {
    if (4 * i + 3 < nval) {
      reinterpret_cast<v4i*>(sc_b + kbase)[i] = reinterpret_cast<const v4i*>(sc_stage)[i];
    } else {
      for (int e = 4 * i; e < nval; ++e) sc_b[kbase + e] = sc_stage[e];
    }
  }
  uint32_t* gh = p.hist + (size_t)b * HBINS;
  for (int i = tid; i < HBINS; i += DS_NT) {
    const uint32_t v = hist[i];
    if (v) atomicAdd(&gh[i], v);
  }
}

// ---------------------------------------------------------------------------
// classify: keys above the k-th bin are selected, keys in it are candidates
// ---------------------------------------------------------------------------

__global__ void __launch_bounds__(CL_NT) decode_classify_kernel(DecodeParams p) {
  __shared__ int wtot[CL_NT / 64];
  __shared__ int bc[2];
  __shared__ int ws_sel[CL_NT / 64], ws_cand[CL_NT / 64];
  __shared__ int base_sel, base_cand;
  const int b = blockIdx.y;
  const int n = seq_len(p, b);
  const int k = p.topk;
  const int c0 = blockIdx.x * CL_CHUNK;
  if (n <= k || c0 >= n) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* sc = p.scores + (size_t)b * p.ld;

  // all of this thread's scores in flight at once
  float v[CL_PER_THREAD];
#pragma unroll
  for (int i = 0; i < CL_PER_THREAD / 4; ++i) {
    const int j = c0 + 4 * (tid + i * CL_NT);
    v4i x = v4i{0, 0, 0, 0};
    if (j + 3 < n) {
      x = *reinterpret_cast<const v4i*>(sc + j);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (j + e < n) x[e] = __float_as_int(sc[j + e]);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) v[4 * i + e] = __int_as_float(x[e]);
  }
  kth_bin<CL_NT>(p.hist + (size_t)b * HBINS, k, wtot, bc);
  const uint32_t dstar = (uint32_t)bc[0];

  int nsel = 0, ncand = 0;
#pragma unroll
  for (int i = 0; i < CL_PER_THREAD; ++i) {
    const int j = c0 + 4 * (tid + (i >> 2) * CL_NT) + (i & 3);
    const uint32_t dg = ordered_key(v[i]) >> 20;
    nsel += (j < n && dg > dstar);
    ncand += (j < n && dg == dstar);
  }
  // one atomic per workgroup and list
  int s_incl = nsel, c_incl = ncand;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int a = __shfl_up(s_incl, o), c = __shfl_up(c_incl, o);
    if (lane >= o) {
      s_incl += a;
      c_incl += c;
    }
  }
  if (lane == 63) {
    ws_sel[wave] = s_incl;
    ws_cand[wave] = c_incl;
  }
  __syncthreads();
  int s_pre = s_incl - nsel, c_pre = c_incl - ncand, s_tot = 0, c_tot = 0;
#pragma unroll
  for (int w = 0; w < CL_NT / 64; ++w) {
    s_pre += (w < wave) ? ws_sel[w] : 0;
    c_pre += (w < wave) ? ws_cand[w] : 0;
    s_tot += ws_sel[w];
    c_tot += ws_cand[w];
  }
  if (tid == 0) {
    base_sel = s_tot ? atomicAdd(&p.counts[2 * b], s_tot) : 0;
    base_cand = c_tot ? atomicAdd(&p.counts[2 * b + 1], c_tot) : 0;
  }
  __syncthreads();
  int* sel = p.sel_idx + (size_t)b * p.topk;
  uint32_t* ckey = p.cand_key + (size_t)b * p.Lmax;
  int* cidx = p.cand_idx + (size_t)b * p.Lmax;
  int ps = base_sel + s_pre, pc = base_cand + c_pre;
#pragma unroll
  for (int i = 0; i < CL_PER_THREAD; ++i) {
    const int j = c0 + 4 * (tid + (i >> 2) * CL_NT) + (i & 3);
    const uint32_t key = ordered_key(v[i]);
    const uint32_t dg = key >> 20;
    if (j < n && dg > dstar) {
      sel[ps++] = j;
    } else if (j < n && dg == dstar) {
      ckey[pc] = key;
      cidx[pc] = j;
      ++pc;
    }
  }
}

// ---------------------------------------------------------------------------
// finalize: exact choice among the candidates, ascending output
// ---------------------------------------------------------------------------

namespace {

struct FinShared {
  int wtot[FN_NT / 64];
  uint32_t hist8[256];
  int bc[4];
};

// exclusive scan of v over the workgroup; *total gets the sum
__device__ int fn_scan(int v, FinShared& sh, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  if (lane == 63) sh.wtot[wave] = incl;
  __syncthreads();
  int pre = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < FN_NT / 64; ++w) {
    const int x = sh.wtot[w];
    pre += (w < wave) ? x : 0;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return pre + incl - v;
}

}  // namespace

__global__ void __launch_bounds__(FN_NT) decode_finalize_kernel(DecodeParams p) {
  extern __shared__ uint32_t dyn[];
  __shared__ FinShared sh;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int n = seq_len(p, b);
  const int k = p.topk;
  int* out = p.out_idx + (size_t)b * k;
  float* osc = p.out_score ? p.out_score + (size_t)b * k : nullptr;
  const float* sc = p.scores + (size_t)b * p.ld;

  if (n <= k) {
    for (int j = tid; j < k; j += FN_NT) {
      out[j] = j < n ? j : -1;
      if (osc) osc[j] = j < n ? sc[j] : -__builtin_inff();
    }
    return;
  }
  const int nw = (p.Lmax + 31) >> 5;
  uint32_t* bm = dyn;                 // selected keys
  uint32_t* tb = dyn + nw;            // keys tied with the k-th score
  uint32_t* lkey = dyn + 2 * nw;      // candidate keys (when they fit)
  for (int i = tid; i < 2 * nw; i += FN_NT) dyn[i] = 0u;
  const int n_sel = p.counts[2 * b];
  const int m = p.counts[2 * b + 1];
  int need = k - n_sel;                // keys still to take from the candidates (>= 1)
  const uint32_t* gkey = p.cand_key + (size_t)b * p.Lmax;
  const int* gidx = p.cand_idx + (size_t)b * p.Lmax;
  const bool in_lds = m <= FN_CAP;
  if (in_lds)
    for (int c = tid; c < m; c += FN_NT) lkey[c] = gkey[c];
  __syncthreads();
  const int* sel = p.sel_idx + (size_t)b * p.topk;
  for (int i = tid; i < n_sel; i += FN_NT) {
    const int j = sel[i];
    atomicOr(&bm[j >> 5], 1u << (j & 31));
  }
  const uint32_t* keys = in_lds ? lkey : gkey;

  // exact k-th key among the candidates: they share the top 12 bits
  uint32_t prefix = m ? keys[0] & 0xFFF00000u : 0u;
  uint32_t pmask = 0xFFF00000u;
  for (int bit = 19; bit >= 0;) {
    const int nb = bit + 1 < 8 ? bit + 1 : 8;
    const int shift = bit + 1 - nb;
    const uint32_t dm = (1u << nb) - 1u;
    for (int i = tid; i < 256; i += FN_NT) sh.hist8[i] = 0u;
    __syncthreads();
    for (int c = tid; c < m; c += FN_NT) {
      const uint32_t key = keys[c];
      if ((key & pmask) == prefix) atomicAdd(&sh.hist8[(key >> shift) & dm], 1u);
    }
    __syncthreads();
    const int hv = tid < 256 ? (int)sh.hist8[tid] : 0;
    int t2;
    const int pre = fn_scan(hv, sh, &t2);
    const int ab = t2 - pre - hv;      // entries in higher bins
    if (tid < 256 && ab < need && ab + hv >= need) {
      sh.bc[0] = tid;
      sh.bc[1] = ab;
    }
    __syncthreads();
    prefix |= (uint32_t)sh.bc[0] << shift;
    pmask |= dm << shift;
    need -= sh.bc[1];
    bit -= nb;
    __syncthreads();
  }
  const uint32_t kstar = prefix;
  for (int c = tid; c < m; c += FN_NT) {
    const uint32_t key = keys[c];
    const int j = gidx[c];
    if (key > kstar) atomicOr(&bm[j >> 5], 1u << (j & 31));
    else if (key == kstar) atomicOr(&tb[j >> 5], 1u << (j & 31));
  }
  __syncthreads();

  // ties: the `need` lowest indices
  const int wpt = (nw + FN_NT - 1) / FN_NT;   // words per thread, contiguous
  {
    int c = 0;
    for (int i = 0; i < wpt; ++i) {
      const int wd = tid * wpt + i;
      if (wd < nw) c += __popc(tb[wd]);
    }
    int t3;
    int before = fn_scan(c, sh, &t3);
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
  __syncthreads();

  // write the selection in ascending key order
  {
    int c = 0;
    for (int i = 0; i < wpt; ++i) {
      const int wd = tid * wpt + i;
      if (wd < nw) c += __popc(bm[wd]);
    }
    int t4;
    int pos = fn_scan(c, sh, &t4);
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

__global__ void decode_prepare_kernel(uint32_t* hist, int nh, int* counts, int nc) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < nh; i += gridDim.x * blockDim.x) hist[i] = 0u;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < nc; i += gridDim.x * blockDim.x) counts[i] = 0;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

size_t decode_finalize_lds_bytes(int Lmax) {
  const size_t nw = ((size_t)Lmax + 31) / 32;
  return (2 * nw + (size_t)FN_CAP) * sizeof(uint32_t);
}

bool decode_supported(int H, int D, int Lmax) {
  if (!(H == 16 || H == 32 || H == 64)) return false;
  if (D != 64 && D != 128) return false;
  return decode_finalize_lds_bytes(Lmax) <= 150 * 1024;
}

int decode_hist_bins() { return HBINS; }

template <int H, int D>
static void launch_score(const DecodeParams& p, hipStream_t stream) {
  dim3 grid((p.Lmax + DS_KPB - 1) / DS_KPB, p.B);
  hipLaunchKernelGGL((decode_score_kernel<H, D>), grid, dim3(DS_NT), 0, stream, p);
}

hipError_t decode_launch(const DecodeParams& p, int H, int D, hipStream_t stream) {
  const int nh = p.B * HBINS;
  const int pg = (nh + 255) / 256 < 1024 ? (nh + 255) / 256 : 1024;
  hipLaunchKernelGGL(decode_prepare_kernel, dim3(pg), dim3(256), 0, stream, p.hist, nh, p.counts, 2 * p.B);
  if (H == 64 && D == 128) launch_score<64, 128>(p, stream);
  else if (H == 64 && D == 64) launch_score<64, 64>(p, stream);
  else if (H == 32 && D == 128) launch_score<32, 128>(p, stream);
  else if (H == 32 && D == 64) launch_score<32, 64>(p, stream);
  else if (H == 16 && D == 128) launch_score<16, 128>(p, stream);
  else if (H == 16 && D == 64) launch_score<16, 64>(p, stream);
  else return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_classify_kernel, dim3((p.Lmax + CL_CHUNK - 1) / CL_CHUNK, p.B), dim3(CL_NT), 0, stream,
                     p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = decode_finalize_lds_bytes(p.Lmax);
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(decode_finalize_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_finalize_kernel, dim3(p.B), dim3(FN_NT), lds, stream, p);
  return hipGetLastError();
}

}  // namespace dsa
