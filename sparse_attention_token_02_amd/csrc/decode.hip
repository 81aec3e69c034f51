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
// decode_score_kernel streams the fp8 cache once with 16-byte loads; a wave
// reads 32 whole consecutive keys per step.  Each lane owns one key column and
// the D/2 contiguous bytes of its half of that key; fp8 is widened to bf16 exactly (e4m3 is a subset of bf16) and the
// contraction runs on v_mfma_f32_32x32x16_bf16 with the heads on the MFMA row
// dimension (q stays in registers).  The per-token fp32 scale is applied to
// the fp32 score, never folded into the bf16 operand (that product would not
// be exact).  Scores go to a workspace row, and a 4096-bin histogram of the
// top 12 bits of their order-preserving keys is accumulated per sequence.
//
// decode_select_kernel (one workgroup per sequence) reads the histogram to
// find the bin of the k-th score, marks every key of a higher bin in an LDS
// bitmap, gathers the keys of that bin as candidates, finishes the exact
// selection among them (radix select, ties to the lower index) and writes the
// selected keys in ascending order by a prefix scan over the bitmap.
#include "device_common.hpp"
#include "kernels.hpp"

namespace dsa {

namespace {

constexpr int DS_NT = 256;          // score kernel threads
constexpr int DS_NSUB = 8;          // 32-key subtiles per wave
constexpr int DS_KPB = (DS_NT / 64) * DS_NSUB * 32;   // keys per workgroup
constexpr int SEL_NT = 1024;        // select kernel threads
constexpr int SEL_CAP = 4096;       // LDS candidates of the threshold bin
constexpr int HBINS = 4096;

// two e4m3 (bytes 2*HI, 2*HI+1 of src) -> two bf16, exact
template <bool HI>
__device__ __forceinline__ uint32_t cvt2(uint32_t src) {
  auto r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(src, 1.0f, HI);
  return __builtin_bit_cast(uint32_t, r);
}

}  // namespace

template <int H, int D>
__global__ void __launch_bounds__(DS_NT, 2) decode_score_kernel(DecodeParams p) {
  constexpr int MB = (H + 31) / 32;
  constexpr int KS = D / 16;              // bf16 MFMA steps along D
  constexpr int HALF = D / 2;             // fp8 bytes of one key half
  constexpr int NLD = HALF / 16;          // 16-byte loads per lane per key
  __shared__ uint32_t hist[HBINS];

  const int b = blockIdx.y;
  const int len = min(max(p.lens[b], 0), p.Lmax);   // lengths outside [0, Lmax] are clamped
  const int kbase = blockIdx.x * DS_KPB;
  if (kbase >= len) return;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int kh = lane >> 5;
  const int col = lane & 31;

  for (int i = tid; i < HBINS; i += DS_NT) hist[i] = 0u;

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
  __syncthreads();

  const uint8_t* cache_b = p.cache + (size_t)b * p.Lmax * D;
  const float* ks_b = p.k_scale + (size_t)b * p.Lmax;
  float* sc_b = p.scores + (size_t)b * p.Lmax;
  const int wbase = kbase + wave * DS_NSUB * 32;

  v4i raw[NLD];
  float ksc = 0.f;
  auto fetch = [&](int s0) {
    const int s = s0 + col;
#pragma unroll
    for (int i = 0; i < NLD; ++i) raw[i] = v4i{0, 0, 0, 0};
    ksc = 0.f;
    if (s < len) {
#pragma unroll
      for (int i = 0; i < NLD; ++i)
        raw[i] = *reinterpret_cast<const v4i*>(cache_b + (size_t)s * D + kh * HALF + 16 * i);
      ksc = ks_b[s];
    }
  };

  if (wbase < len) fetch(wbase);
#pragma unroll 1
  for (int sub = 0; sub < DS_NSUB; ++sub) {
    const int s0 = wbase + 32 * sub;
    if (s0 >= len) break;
    v4i cur[NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i) cur[i] = raw[i];
    const float cks = ksc;
    if (sub + 1 < DS_NSUB && s0 + 32 < len) fetch(s0 + 32);

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
      sc_b[s] = score;
      atomicAdd(&hist[ordered_key(score) >> 20], 1u);
    }
  }
  __syncthreads();
  uint32_t* gh = p.hist + (size_t)b * HBINS;
  for (int i = tid; i < HBINS; i += DS_NT) {
    const uint32_t v = hist[i];
    if (v) atomicAdd(&gh[i], v);
  }
}

// ---------------------------------------------------------------------------
// select
// ---------------------------------------------------------------------------

namespace {

struct SelShared {
  int wtot[SEL_NT / 64];
  uint32_t hist8[256];
  int bcast[4];
  int cand_cnt;
};

// exclusive scan of v over the workgroup; *total gets the sum
__device__ int sel_scan(int v, SelShared& sh, int* total) {
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
  for (int w = 0; w < SEL_NT / 64; ++w) {
    const int x = sh.wtot[w];
    pre += (w < wave) ? x : 0;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return pre + incl - v;
}

// suffix scan: sum of v over threads with a larger index; *total gets the sum
__device__ int sel_suffix(int v, SelShared& sh, int* total) {
  int tot;
  const int pre = sel_scan(v, sh, &tot);
  *total = tot;
  return tot - pre - v;
}

}  // namespace

__global__ void __launch_bounds__(SEL_NT) decode_select_kernel(DecodeParams p) {
  extern __shared__ uint32_t dyn[];
  __shared__ SelShared sh;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int n = min(max(p.lens[b], 0), p.Lmax);
  const int k = p.topk;
  int* out = p.out_idx + (size_t)b * k;
  float* osc = p.out_score ? p.out_score + (size_t)b * k : nullptr;
  const float* sc = p.scores + (size_t)b * p.Lmax;

  if (n <= k) {
    for (int j = tid; j < k; j += SEL_NT) {
      out[j] = j < n ? j : -1;
      if (osc) osc[j] = j < n ? sc[j] : -__builtin_inff();
    }
    return;
  }
  const int nw = (p.Lmax + 31) >> 5;
  uint32_t* bm = dyn;                 // selected keys
  uint32_t* tb = dyn + nw;            // keys tied with the k-th score
  uint32_t* ckey = dyn + 2 * nw;      // candidate keys
  int* cidx = reinterpret_cast<int*>(dyn + 2 * nw + SEL_CAP);

  // ---- bin of the k-th score from the histogram (4 bins per thread)
  const uint32_t* gh = p.hist + (size_t)b * HBINS;
  uint32_t h[4];
  int s4 = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = gh[4 * tid + i];
    s4 += (int)h[i];
  }
  int tot;
  int above = sel_suffix(s4, sh, &tot);
#pragma unroll
  for (int i = 3; i >= 0; --i) {
    if (above < k && above + (int)h[i] >= k) {
      sh.bcast[0] = 4 * tid + i;
      sh.bcast[1] = above;
    }
    above += (int)h[i];
  }
  for (int i = tid; i < 2 * nw; i += SEL_NT) dyn[i] = 0u;
  if (tid == 0) sh.cand_cnt = 0;
  __syncthreads();
  const uint32_t dstar = (uint32_t)sh.bcast[0];
  int need = k - sh.bcast[1];

  // ---- classify every key
  for (int j = tid; j < n; j += SEL_NT) {
    const uint32_t key = ordered_key(sc[j]);
    const uint32_t dg = key >> 20;
    if (dg > dstar) {
      atomicOr(&bm[j >> 5], 1u << (j & 31));
    } else if (dg == dstar) {
      const int pos = atomicAdd(&sh.cand_cnt, 1);
      if (pos < SEL_CAP) {
        ckey[pos] = key;
        cidx[pos] = j;
      }
    }
  }
  __syncthreads();
  const int m = sh.cand_cnt;
  const bool in_lds = m <= SEL_CAP;

  // ---- exact k-th key among the bin: 8, 8 and 4 more bits
  uint32_t prefix = dstar << 20, pmask = 0xFFF00000u;
  for (int bit = 19; bit >= 0;) {
    const int nb = bit + 1 < 8 ? bit + 1 : 8;
    const int shift = bit + 1 - nb;
    const uint32_t dm = (1u << nb) - 1u;
    for (int i = tid; i < 256; i += SEL_NT) sh.hist8[i] = 0u;
    __syncthreads();
    if (in_lds) {
      for (int c = tid; c < m; c += SEL_NT) {
        const uint32_t key = ckey[c];
        if ((key & pmask) == prefix) atomicAdd(&sh.hist8[(key >> shift) & dm], 1u);
      }
    } else {
      for (int j = tid; j < n; j += SEL_NT) {
        const uint32_t key = ordered_key(sc[j]);
        if ((key & pmask) == prefix) atomicAdd(&sh.hist8[(key >> shift) & dm], 1u);
      }
    }
    __syncthreads();
    // 256 bins: the first 256 threads hold one each
    const int hv = tid < 256 ? (int)sh.hist8[tid] : 0;
    int t2;
    const int ab = sel_suffix(hv, sh, &t2);
    if (tid < 256 && ab < need && ab + hv >= need) {
      sh.bcast[2] = tid;
      sh.bcast[3] = ab;
    }
    __syncthreads();
    prefix |= (uint32_t)sh.bcast[2] << shift;
    pmask |= dm << shift;
    need -= sh.bcast[3];
    bit -= nb;
    __syncthreads();
  }
  const uint32_t kstar = prefix;   // exact k-th key; `need` keys equal to it are taken

  // ---- mark the bin's keys above kstar, and the ties
  if (in_lds) {
    for (int c = tid; c < m; c += SEL_NT) {
      const uint32_t key = ckey[c];
      const int j = cidx[c];
      if (key > kstar) atomicOr(&bm[j >> 5], 1u << (j & 31));
      else if (key == kstar) atomicOr(&tb[j >> 5], 1u << (j & 31));
    }
  } else {
    for (int j = tid; j < n; j += SEL_NT) {
      const uint32_t key = ordered_key(sc[j]);
      if ((key >> 20) != dstar) continue;
      if (key > kstar) atomicOr(&bm[j >> 5], 1u << (j & 31));
      else if (key == kstar) atomicOr(&tb[j >> 5], 1u << (j & 31));
    }
  }
  __syncthreads();

  // ---- ties: the `need` lowest indices
  const int wpt = (nw + SEL_NT - 1) / SEL_NT;   // words per thread, contiguous
  {
    int c = 0;
    for (int i = 0; i < wpt; ++i) {
      const int wd = tid * wpt + i;
      if (wd < nw) c += __popc(tb[wd]);
    }
    int t3;
    int before = sel_scan(c, sh, &t3);
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

  // ---- write the selection in ascending key order
  {
    int c = 0;
    for (int i = 0; i < wpt; ++i) {
      const int wd = tid * wpt + i;
      if (wd < nw) c += __popc(bm[wd]);
    }
    int t4;
    int pos = sel_scan(c, sh, &t4);
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

__global__ void decode_prepare_kernel(uint32_t* hist, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) hist[i] = 0u;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

bool decode_supported(int H, int D, int Lmax) {
  if (!(H == 16 || H == 32 || H == 64)) return false;
  if (D != 64 && D != 128) return false;
  return decode_select_lds_bytes(Lmax) <= 150 * 1024;
}

size_t decode_select_lds_bytes(int Lmax) {
  const size_t nw = ((size_t)Lmax + 31) / 32;
  return (2 * nw + 2 * (size_t)SEL_CAP) * sizeof(uint32_t);
}

int decode_hist_bins() { return HBINS; }

template <int H, int D>
static void launch_score(const DecodeParams& p, hipStream_t stream) {
  dim3 grid((p.Lmax + DS_KPB - 1) / DS_KPB, p.B);
  hipLaunchKernelGGL((decode_score_kernel<H, D>), grid, dim3(DS_NT), 0, stream, p);
}

hipError_t decode_launch(const DecodeParams& p, int H, int D, hipStream_t stream) {
  const int nh = p.B * HBINS;
  hipLaunchKernelGGL(decode_prepare_kernel, dim3((nh + 255) / 256 < 1024 ? (nh + 255) / 256 : 1024), dim3(256),
                     0, stream, p.hist, nh);
  if (H == 64 && D == 128) launch_score<64, 128>(p, stream);
  else if (H == 64 && D == 64) launch_score<64, 64>(p, stream);
  else if (H == 32 && D == 128) launch_score<32, 128>(p, stream);
  else if (H == 32 && D == 64) launch_score<32, 64>(p, stream);
  else if (H == 16 && D == 128) launch_score<16, 128>(p, stream);
  else if (H == 16 && D == 64) launch_score<16, 64>(p, stream);
  else return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = decode_select_lds_bytes(p.Lmax);
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(decode_select_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_select_kernel, dim3(p.B), dim3(SEL_NT), lds, stream, p);
  return hipGetLastError();
}

}  // namespace dsa
