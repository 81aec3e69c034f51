// C ABI of the lightning-indexer library: argument validation (on the host,
// before anything touches HIP), workspace layout, the IndexCache F/S driver
// and the overlap entry point.  See include/dsa_indexer.h for the contract.
#include <hip/hip_runtime.h>
#include <rocprofiler-sdk-roctx/roctx.h>

#include <cstdarg>
#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "dsa_indexer.h"
#include "kernels.hpp"

namespace {

// A roctx range around one layer of a schedule ("<schedule> layer <l> <F|S>"),
// shown by rocprofv3 --marker-trace; a few ns per layer without a profiler.
struct LayerRange {
  LayerRange(const char* schedule, int layer, char kind) {
    char name[96];
    snprintf(name, sizeof(name), "%s layer %d %c", schedule, layer, kind);
    roctxRangePushA(name);
  }
  ~LayerRange() { roctxRangePop(); }
  LayerRange(const LayerRange&) = delete;
  LayerRange& operator=(const LayerRange&) = delete;
};

}  // namespace

namespace {

thread_local std::string g_err;

dsa_status fail(dsa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

dsa_status ok() {
  g_err.clear();
  return DSA_OK;
}

dsa_status hip_fail(hipError_t e, const char* what) {
  return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr size_t kHeader = 256;          // work counter, kept apart from the lists
constexpr int kMaxSlots = 256;           // persistent workgroups (one per MI355X CU)
constexpr int kMaxTopk = dsa::MAX_TOPK;
constexpr int kMaxDenseL = 16384;
constexpr int kMaxDecodeLmax = 262144;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Layout checks of the workspaces (region order, alignment, total), built in
// with -DDSA_DEBUG_BOUNDS (the sanitizer test builds the host code so); a
// failed check prints where and aborts.
#ifdef DSA_DEBUG_BOUNDS
#define DSA_DCHECK(c)                                                                 \
  do {                                                                                \
    if (!(c)) {                                                                       \
      fprintf(stderr, "DSA_DCHECK failed: %s (%s:%d)\n", #c, __FILE__, __LINE__);   \
      abort();                                                                        \
    }                                                                                 \
  } while (0)
#else
#define DSA_DCHECK(c) ((void)0)
#endif

int prefill_cap(int dt, int H, int D, int topk) { return dsa::prefill_list_capacity(dt, H, D, topk); }

int prefill_slots(int L, int dt, int H, int D) {
  const int rw = dsa::prefill_rows_per_item(dt, H, D);
  const int items = (L + rw - 1) / rw;
  return items < kMaxSlots ? items : kMaxSlots;
}

size_t prefill_ws_bytes(int L, int H, int D, int topk, dsa_dtype dt) {
  const int slots = prefill_slots(L, (int)dt, H, D);
  const size_t per = (size_t)dsa::prefill_rows_per_item((int)dt, H, D) * prefill_cap((int)dt, H, D, topk);
  const size_t lists = align_up((size_t)slots * per * 4, 256);
  DSA_DCHECK(per > 0 && slots >= 1 && slots <= kMaxSlots);
  DSA_DCHECK(kHeader % 256 == 0 && lists >= (size_t)slots * per * 4);
  return kHeader + 2 * lists;
}

dsa_status check_prefill_shape(int L, int H, int D, int topk, dsa_dtype dt) {
  if (dt != DSA_BF16 && dt != DSA_FP8_E4M3) return fail(DSA_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
  if (L < 1) return fail(DSA_ERR_INVALID_ARG, "L must be >= 1 (got %d)", L);
  if (topk < 1 || topk > kMaxTopk) return fail(DSA_ERR_INVALID_ARG, "topk must be in [1, %d] (got %d)", kMaxTopk, topk);
  if (H < 1 || D < 1) return fail(DSA_ERR_INVALID_ARG, "H and D must be positive");
  if (!dsa::prefill_supported((int)dt, H, D))
    return fail(DSA_ERR_UNSUPPORTED, "prefill kernels are not built for dt=%d H=%d D=%d", (int)dt, H, D);
  if (prefill_cap((int)dt, H, D, topk) == 0)
    return fail(DSA_ERR_UNSUPPORTED, "topk=%d does not fit the candidate lists in LDS for H=%d D=%d", topk, H, D);
  return DSA_OK;
}

int device_cus(int* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  *out = cus;
  return 0;
}

struct PrefillArgs {
  const void* q;
  const float* q_scale;
  int64_t qs_head_stride;
  const void* k;
  const float* k_scale;
  const uint16_t* w;
  int L, H, D, topk;           // L: query rows
  dsa_dtype dt;
  int32_t* out_idx;
  float* out_score;
  float* out_dense;
  void* ws;
  size_t ws_bytes;
  hipStream_t stream;
  int q0 = 0;                  // absolute position of query row 0; keys are q0 + L
};

dsa_status validate_prefill(const PrefillArgs& a, bool check_dense = true) {
  dsa_status st = check_prefill_shape(a.L, a.H, a.D, a.topk, a.dt);
  if (st != DSA_OK) return st;
  if (!a.q || !a.k || !a.w || !a.out_idx) return fail(DSA_ERR_INVALID_ARG, "q, k, w and out_idx must not be NULL");
  if (!aligned16(a.q) || !aligned16(a.k)) return fail(DSA_ERR_INVALID_ARG, "q and k must be 16-byte aligned");
  if (a.qs_head_stride != 0 && a.qs_head_stride != 1)
    return fail(DSA_ERR_INVALID_ARG, "q_scale_head_stride must be 0 or 1");
  if (check_dense && a.out_dense && a.L > kMaxDenseL)
    return fail(DSA_ERR_INVALID_ARG, "out_dense_score is only allowed for L <= %d", kMaxDenseL);
  const size_t need = prefill_ws_bytes(a.L, a.H, a.D, a.topk, a.dt);
  if (!a.ws || a.ws_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, a.ws ? a.ws_bytes : (size_t)0);
  if (!aligned16(a.ws)) return fail(DSA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  return DSA_OK;
}

dsa_status launch_prefill(const PrefillArgs& a) {
  int cus = 0;
  if (device_cus(&cus) != 0) return fail(DSA_ERR_HIP, "no HIP device");
  dsa::PrefillParams p{};
  p.q = static_cast<const uint8_t*>(a.q);
  p.q_scale = a.q_scale;
  p.qs_row = a.qs_head_stride ? a.H : 1;
  p.hr = a.H;
  p.qs_head = a.qs_head_stride;
  p.k = static_cast<const uint8_t*>(a.k);
  p.k_scale = a.k_scale;
  p.w = a.w;
  p.L = a.q0 + a.L;
  p.q0 = a.q0;
  p.topk = a.topk;
  p.cap = prefill_cap((int)a.dt, a.H, a.D, a.topk);
  p.sample_m = dsa::prefill_sample_keys((int)a.dt, a.H, a.D);
  p.out_idx = a.out_idx;
  p.out_score = a.out_score;
  p.out_dense = a.out_dense;
  const int rw = dsa::prefill_rows_per_item((int)a.dt, a.H, a.D);
  p.n_items = (a.L + rw - 1) / rw;
  const int slots = prefill_slots(a.L, (int)a.dt, a.H, a.D);
  uint8_t* base = static_cast<uint8_t*>(a.ws);
  p.counter = reinterpret_cast<int*>(base);
  const size_t lst = align_up((size_t)slots * rw * p.cap * 4, 256);
  p.ws_sc = reinterpret_cast<float*>(base + kHeader);
  p.ws_ix = reinterpret_cast<int32_t*>(base + kHeader + lst);
  const int grid = slots < cus ? slots : cus;
  hipError_t e = dsa::prefill_launch(p, (int)a.dt, a.H, a.D, grid, a.stream);
  if (e != hipSuccess) return hip_fail(e, "prefill launch");
  return DSA_OK;
}

// Decode workspace: per score workgroup of each sequence, its packed
// histograms, its list's cut (lowest bin kept, entries) and its list of
// (key, index) candidates.
struct DecodeWs {
  size_t hdr, hist, wgcut, cand, total;
};

DecodeWs decode_ws(int B, int Lmax) {
  DecodeWs w{};
  const dsa::DecodeWsSizes z = dsa::decode_ws_sizes(Lmax);
  size_t off = 0;
  w.hdr = off;   // per-sequence header at a fixed place: its words outlive calls of other sizes
  off += align_up((size_t)B * sizeof(dsa::DecodeHdr), 256);
  w.hist = off;
  off += align_up((size_t)B * z.hist_words * 4, 256);
  w.wgcut = off;
  off += align_up((size_t)B * z.nwg * 8, 256);
  w.cand = off;
  off += align_up((size_t)B * z.cand_entries * 8, 256);
  w.total = off;
  DSA_DCHECK(w.hdr == 0 && w.hdr + (size_t)B * sizeof(dsa::DecodeHdr) <= w.hist);
  DSA_DCHECK(w.hist % 256 == 0 && w.hist + (size_t)B * z.hist_words * 4 <= w.wgcut);
  DSA_DCHECK(w.wgcut % 256 == 0 && w.wgcut + (size_t)B * z.nwg * 8 <= w.cand);
  DSA_DCHECK(w.cand % 256 == 0 && w.cand + (size_t)B * z.cand_entries * 8 <= w.total);
  return w;
}

size_t decode_ws_bytes(int B, int Lmax) { return decode_ws(B, Lmax).total; }

// A fresh 32-bit value per decode launch (SplitMix64 of a process-wide
// counter started from the clock), for the tag of the sequences' pool counters.
uint32_t next_nonce() {
  static std::atomic<uint64_t> ctr{(uint64_t)std::chrono::steady_clock::now().time_since_epoch().count()};
  uint64_t z = ctr.fetch_add(0x9E3779B97F4A7C15ull) + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return (uint32_t)(z ^ (z >> 31));
}

struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* w;
  const uint8_t* cache;
  const float* k_scale;
  const int32_t* lens;
  int B, Lmax, H, D, topk;
  int32_t* out_idx;
  float* out_score;
  void* ws;
  size_t ws_bytes;
  hipStream_t stream;
  // paged cache: Lmax = max_blocks * page_size
  const int32_t* block_table = nullptr;
  int max_blocks = 0, page_size = 0, num_pages = 0;
};

dsa_status validate_decode(const DecodeArgs& a) {
  if (a.B < 1 || a.Lmax < 1 || a.topk < 1 || a.topk > kMaxTopk || a.H < 1 || a.D < 1)
    return fail(DSA_ERR_INVALID_ARG, "bad decode sizes B=%d Lmax=%d H=%d D=%d topk=%d", a.B, a.Lmax, a.H, a.D,
                a.topk);
  if (a.Lmax > kMaxDecodeLmax || !dsa::decode_supported(a.H, a.D, a.Lmax))
    return fail(DSA_ERR_UNSUPPORTED, "decode kernels are not built for H=%d D=%d Lmax=%d", a.H, a.D, a.Lmax);
  if (!a.q || !a.w || !a.cache || !a.k_scale || !a.lens || !a.out_idx)
    return fail(DSA_ERR_INVALID_ARG, "q, w, k_cache, k_scale, seq_lens and out_idx must not be NULL");
  if (!aligned16(a.q) || !aligned16(a.cache)) return fail(DSA_ERR_INVALID_ARG, "q and k_cache must be 16-byte aligned");
  const size_t need = decode_ws_bytes(a.B, a.Lmax);
  if (!a.ws || a.ws_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, a.ws ? a.ws_bytes : (size_t)0);
  if (!aligned16(a.ws)) return fail(DSA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  return DSA_OK;
}

dsa_status launch_decode(const DecodeArgs& a) {
  dsa::DecodeParams p{};
  p.q = a.q;
  p.w = a.w;
  p.hr = a.H;
  p.cache = a.cache;
  p.k_scale = a.k_scale;
  p.lens = a.lens;
  p.B = a.B;
  p.Lmax = a.Lmax;
  p.topk = a.topk;
  p.out_idx = a.out_idx;
  p.out_score = a.out_score;
  uint8_t* base = static_cast<uint8_t*>(a.ws);
  const DecodeWs lay = decode_ws(a.B, a.Lmax);
  p.hdr = reinterpret_cast<dsa::DecodeHdr*>(base + lay.hdr);
  p.nonce = next_nonce();
  p.hist = reinterpret_cast<uint32_t*>(base + lay.hist);
  p.wgcut = reinterpret_cast<int2*>(base + lay.wgcut);
  p.cand = reinterpret_cast<uint2*>(base + lay.cand);
  p.block_table = a.block_table;
  p.max_blocks = a.max_blocks;
  p.page_shift = a.page_size > 0 ? __builtin_ctz((unsigned)a.page_size) : 0;
  p.num_pages = a.num_pages;
  hipError_t e = dsa::decode_launch(p, a.H, a.D, a.stream);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return DSA_OK;
}

// Events of one call; destroyed on return (a pending event is released by
// the runtime once it completes).
struct EventSet {
  hipEvent_t ev[4] = {};
  int n = 0;
  ~EventSet() {
    for (int i = 0; i < n; ++i) (void)hipEventDestroy(ev[i]);
  }
  hipError_t create(int count, unsigned flags) {
    for (; n < count; ++n) {
      hipError_t e = hipEventCreateWithFlags(&ev[n], flags);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
};

}  // namespace

extern "C" {

const char* dsa_last_error(void) { return g_err.c_str(); }

int dsa_abi_version(void) { return 1; }

dsa_status dsa_indexer_topk_prefill_workspace(int L, int H, int D, int topk, dsa_dtype dt, size_t* bytes) {
  if (!bytes) return fail(DSA_ERR_INVALID_ARG, "bytes must not be NULL");
  dsa_status st = check_prefill_shape(L, H, D, topk, dt);
  if (st != DSA_OK) return st;
  *bytes = prefill_ws_bytes(L, H, D, topk, dt);
  return ok();
}

dsa_status dsa_indexer_topk_prefill(const void* q, const float* q_scale, int64_t q_scale_head_stride,
                                    const void* k, const float* k_scale, const uint16_t* w, int L, int H,
                                    int D, int topk, dsa_dtype dt, int32_t* out_idx, float* out_topk_score,
                                    float* out_dense_score, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  PrefillArgs a{q, q_scale, q_scale_head_stride, k, k_scale, w, L, H, D, topk, dt, out_idx,
                out_topk_score, out_dense_score, workspace, workspace_bytes,
                static_cast<hipStream_t>(stream)};
  dsa_status st = validate_prefill(a);
  if (st != DSA_OK) return st;
  st = launch_prefill(a);
  if (st != DSA_OK) return st;
  return ok();
}

dsa_status dsa_indexer_topk_prefill_chunk(const void* q, const float* q_scale, int64_t q_scale_head_stride,
                                          const void* k, const float* k_scale, const uint16_t* w, int q_offset,
                                          int Lq, int H, int D, int topk, dsa_dtype dt, int32_t* out_idx,
                                          float* out_topk_score, void* workspace, size_t workspace_bytes,
                                          void* stream) {
  if (q_offset < 0) return fail(DSA_ERR_INVALID_ARG, "q_offset must be >= 0 (got %d)", q_offset);
  if (Lq >= 1 && q_offset > INT32_MAX - Lq)
    return fail(DSA_ERR_INVALID_ARG, "q_offset + Lq must fit in int32");
  PrefillArgs a{q, q_scale, q_scale_head_stride, k, k_scale, w, Lq, H, D, topk, dt, out_idx,
                out_topk_score, nullptr, workspace, workspace_bytes, static_cast<hipStream_t>(stream)};
  a.q0 = q_offset;
  dsa_status st = validate_prefill(a);
  if (st != DSA_OK) return st;
  st = launch_prefill(a);
  if (st != DSA_OK) return st;
  return ok();
}

// Ragged batch workspace: header (work counter at 0, item count at 128), the
// item table (int4 per item), then the candidate lists of every slot.
struct VarlenWs {
  size_t items, lists, total;
  int cap_items, slots;
};

static bool varlen_ws(int nseq, int total_q, int H, int D, int topk, dsa_dtype dt, VarlenWs* w) {
  const int rw = dsa::prefill_rows_per_item((int)dt, H, D);
  const int64_t cap = ((int64_t)total_q + rw - 1) / rw + nseq;
  if (cap > INT32_MAX / 2) return false;
  w->cap_items = (int)cap;
  w->slots = w->cap_items < kMaxSlots ? w->cap_items : kMaxSlots;
  if (w->slots < 1) w->slots = 1;
  w->items = kHeader;
  w->lists = w->items + align_up((size_t)w->cap_items * 16, 256);
  const size_t per = (size_t)rw * prefill_cap((int)dt, H, D, topk);
  w->total = w->lists + 2 * align_up((size_t)w->slots * per * 4, 256);
  DSA_DCHECK(w->items == kHeader && w->items + (size_t)w->cap_items * 16 <= w->lists && w->lists % 256 == 0);
  DSA_DCHECK(w->slots >= 1 && w->slots <= kMaxSlots && w->lists + 2 * (size_t)w->slots * per * 4 <= w->total);
  return true;
}

dsa_status dsa_indexer_topk_prefill_varlen_workspace(int nseq, int total_q, int H, int D, int topk, dsa_dtype dt,
                                                     size_t* bytes) {
  if (!bytes) return fail(DSA_ERR_INVALID_ARG, "bytes must not be NULL");
  if (nseq < 1 || total_q < 0) return fail(DSA_ERR_INVALID_ARG, "nseq must be >= 1 and total_q >= 0");
  dsa_status st = check_prefill_shape(1, H, D, topk, dt);
  if (st != DSA_OK) return st;
  VarlenWs w;
  if (!varlen_ws(nseq, total_q, H, D, topk, dt, &w)) return fail(DSA_ERR_INVALID_ARG, "batch too large");
  *bytes = w.total;
  return ok();
}

dsa_status dsa_indexer_topk_prefill_varlen(const void* q, const float* q_scale, int64_t q_scale_head_stride,
                                           const void* k, const float* k_scale, const uint16_t* w,
                                           const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int nseq,
                                           int total_q, int total_k, int H, int D, int topk, dsa_dtype dt,
                                           int32_t* out_idx, float* out_topk_score, void* workspace,
                                           size_t workspace_bytes, void* stream) {
  size_t need = 0;
  dsa_status st = dsa_indexer_topk_prefill_varlen_workspace(nseq, total_q, H, D, topk, dt, &need);
  if (st != DSA_OK) return st;
  if (total_k < 0) return fail(DSA_ERR_INVALID_ARG, "total_k must be >= 0");
  if (!cu_seqlens_q || !cu_seqlens_k) return fail(DSA_ERR_INVALID_ARG, "cu_seqlens_q and cu_seqlens_k must not be NULL");
  if (total_q == 0 || total_k == 0) return ok();   // nothing to select
  if (!q || !k || !w || !out_idx) return fail(DSA_ERR_INVALID_ARG, "q, k, w and out_idx must not be NULL");
  if (!aligned16(q) || !aligned16(k)) return fail(DSA_ERR_INVALID_ARG, "q and k must be 16-byte aligned");
  if (q_scale_head_stride != 0 && q_scale_head_stride != 1)
    return fail(DSA_ERR_INVALID_ARG, "q_scale_head_stride must be 0 or 1");
  if (!workspace || workspace_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(DSA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  int cus = 0;
  if (device_cus(&cus) != 0) return fail(DSA_ERR_HIP, "no HIP device");
  VarlenWs lay;
  varlen_ws(nseq, total_q, H, D, topk, dt, &lay);
  uint8_t* base = static_cast<uint8_t*>(workspace);
  const int rw = dsa::prefill_rows_per_item((int)dt, H, D);
  dsa::PrefillParams p{};
  p.q = static_cast<const uint8_t*>(q);
  p.q_scale = q_scale;
  p.qs_row = q_scale_head_stride ? H : 1;
  p.hr = H;
  p.qs_head = q_scale_head_stride;
  p.k = static_cast<const uint8_t*>(k);
  p.k_scale = k_scale;
  p.w = w;
  p.topk = topk;
  p.cap = prefill_cap((int)dt, H, D, topk);
  p.sample_m = dsa::prefill_sample_keys((int)dt, H, D);
  p.out_idx = out_idx;
  p.out_score = out_topk_score;
  p.counter = reinterpret_cast<int*>(base);
  p.items = reinterpret_cast<const int4*>(base + lay.items);
  p.n_items_dev = reinterpret_cast<const int*>(base + 128);
  p.ws_sc = reinterpret_cast<float*>(base + lay.lists);
  p.ws_ix = reinterpret_cast<int32_t*>(base + lay.lists + align_up((size_t)lay.slots * rw * p.cap * 4, 256));
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = dsa::prefill_varlen_prepare(cu_seqlens_q, cu_seqlens_k, nseq, total_q, total_k, rw,
                                             reinterpret_cast<int4*>(base + lay.items), reinterpret_cast<int*>(base + 128),
                                             p.counter, s);
  if (e != hipSuccess) return hip_fail(e, "ragged batch prepare");
  const int grid = lay.slots < cus ? lay.slots : cus;
  e = dsa::prefill_launch(p, (int)dt, H, D, grid, s);
  if (e != hipSuccess) return hip_fail(e, "prefill launch");
  return ok();
}

// ---------------------------------------------------------------------------

dsa_status dsa_indexer_topk_decode_workspace(int B, int Lmax, int H, int D, int topk, size_t* bytes) {
  if (!bytes) return fail(DSA_ERR_INVALID_ARG, "bytes must not be NULL");
  if (B < 1 || Lmax < 1 || topk < 1 || topk > kMaxTopk || H < 1 || D < 1)
    return fail(DSA_ERR_INVALID_ARG, "bad decode sizes B=%d Lmax=%d H=%d D=%d topk=%d", B, Lmax, H, D, topk);
  if (Lmax > kMaxDecodeLmax || !dsa::decode_supported(H, D, Lmax))
    return fail(DSA_ERR_UNSUPPORTED, "decode kernels are not built for H=%d D=%d Lmax=%d", H, D, Lmax);
  *bytes = decode_ws_bytes(B, Lmax);
  return ok();
}

dsa_status dsa_indexer_topk_decode(const uint16_t* q, const uint16_t* w, const uint8_t* k_cache,
                                   const float* k_scale, const int32_t* seq_lens, int B, int Lmax, int H, int D,
                                   int topk, int32_t* out_idx, float* out_topk_score, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  DecodeArgs a{q, w, k_cache, k_scale, seq_lens, B, Lmax, H, D, topk, out_idx, out_topk_score, workspace,
               workspace_bytes, static_cast<hipStream_t>(stream)};
  dsa_status st = validate_decode(a);
  if (st != DSA_OK) return st;
  st = launch_decode(a);
  if (st != DSA_OK) return st;
  return ok();
}

dsa_status dsa_indexer_topk_decode_noalloc(const uint16_t* q, const uint16_t* w, const uint8_t* k_cache,
                                           const float* k_scale, const int32_t* seq_lens, int B, int Lmax, int H,
                                           int D, int topk, int32_t* out_idx, float* out_topk_score,
                                           void* stream) {
  if (B < 1 || Lmax < 1 || topk < 1 || topk > kMaxTopk || H < 1 || D < 1)
    return fail(DSA_ERR_INVALID_ARG, "bad decode sizes B=%d Lmax=%d H=%d D=%d topk=%d", B, Lmax, H, D, topk);
  if (Lmax > kMaxDecodeLmax || !dsa::decode_supported(H, D, Lmax))
    return fail(DSA_ERR_UNSUPPORTED, "decode kernels are not built for H=%d D=%d Lmax=%d", H, D, Lmax);
  const size_t need = decode_ws_bytes(B, Lmax);
  if (need > dsa::decode_scratch_bytes())
    return fail(DSA_ERR_UNSUPPORTED,
                "B=%d x Lmax=%d needs %zu bytes of scratch; the allocation-free decode holds %zu "
                "(use dsa_indexer_topk_decode with a workspace)", B, Lmax, need, dsa::decode_scratch_bytes());
  void* scratch = nullptr;
  const hipError_t e = dsa::decode_scratch(&scratch);
  if (e != hipSuccess) return hip_fail(e, "decode scratch address");
  DecodeArgs a{q, w, k_cache, k_scale, seq_lens, B, Lmax, H, D, topk, out_idx, out_topk_score, scratch,
               dsa::decode_scratch_bytes(), static_cast<hipStream_t>(stream)};
  dsa_status st = validate_decode(a);
  if (st != DSA_OK) return st;
  st = launch_decode(a);
  if (st != DSA_OK) return st;
  return ok();
}

dsa_status dsa_indexer_topk_decode_paged(const uint16_t* q, const uint16_t* w, const uint8_t* k_pages,
                                         const float* k_scale_pages, int num_pages, int page_size,
                                         const int32_t* block_table, int max_blocks, const int32_t* seq_lens, int B,
                                         int H, int D, int topk, int32_t* out_idx, float* out_topk_score,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  if (page_size < 32 || (page_size & (page_size - 1)) != 0)
    return fail(DSA_ERR_INVALID_ARG, "page_size must be a power of two >= 32 (got %d)", page_size);
  if (num_pages < 1 || max_blocks < 1)
    return fail(DSA_ERR_INVALID_ARG, "num_pages and max_blocks must be >= 1");
  if ((int64_t)max_blocks * page_size > kMaxDecodeLmax)
    return fail(DSA_ERR_UNSUPPORTED, "max_blocks * page_size must be <= %d", kMaxDecodeLmax);
  if (!block_table) return fail(DSA_ERR_INVALID_ARG, "block_table must not be NULL");
  DecodeArgs a{q, w, k_pages, k_scale_pages, seq_lens, B, max_blocks * page_size, H, D, topk, out_idx,
               out_topk_score, workspace, workspace_bytes, static_cast<hipStream_t>(stream)};
  a.block_table = block_table;
  a.max_blocks = max_blocks;
  a.page_size = page_size;
  a.num_pages = num_pages;
  dsa_status st = validate_decode(a);
  if (st != DSA_OK) return st;
  st = launch_decode(a);
  if (st != DSA_OK) return st;
  return ok();
}

// ---------------------------------------------------------------------------

dsa_status indexcache_resolve(const char* pattern, int N, int32_t* src_layer) {
  if (!pattern) return fail(DSA_ERR_INVALID_ARG, "pattern must not be NULL");
  if (N < 1) return fail(DSA_ERR_INVALID_ARG, "N must be >= 1 (got %d)", N);
  const size_t n = strnlen(pattern, (size_t)N + 1);
  if (n != (size_t)N) return fail(DSA_ERR_INVALID_ARG, "pattern has length %zu, expected N=%d", n, N);
  if (pattern[0] != 'F') return fail(DSA_ERR_INVALID_ARG, "the first layer must be F (got '%c')", pattern[0]);
  int last_f = 0;
  for (int l = 0; l < N; ++l) {
    const char c = pattern[l];
    if (c != 'F' && c != 'S') return fail(DSA_ERR_INVALID_ARG, "pattern[%d] = '%c' is not F or S", l, c);
    if (c == 'F') last_f = l;
    if (src_layer) src_layer[l] = last_f;
  }
  return ok();
}

dsa_status indexcache_run_layers(const char* pattern, int N, const void* const* q, const float* const* q_scale,
                                 int64_t q_scale_head_stride, const void* const* k,
                                 const float* const* k_scale, const uint16_t* const* w, int L, int H, int D,
                                 int topk, dsa_dtype dt, int32_t* tcache, int32_t* src_layer_out,
                                 indexcache_layer_fn hook, void* user, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  std::vector<int32_t> src((size_t)(N > 0 ? N : 1));
  dsa_status st = indexcache_resolve(pattern, N, src.data());
  if (st != DSA_OK) return st;
  if (!q || !k || !w) return fail(DSA_ERR_INVALID_ARG, "q, k and w pointer arrays must not be NULL");
  if (!tcache) return fail(DSA_ERR_INVALID_ARG, "tcache must not be NULL");
  // validate every F layer before enqueueing anything
  for (int l = 0; l < N; ++l) {
    if (pattern[l] != 'F') continue;
    PrefillArgs a{q[l], q_scale ? q_scale[l] : nullptr, q_scale_head_stride, k[l], k_scale ? k_scale[l] : nullptr,
                  w[l], L, H, D, topk, dt, tcache, nullptr, nullptr, workspace, workspace_bytes,
                  static_cast<hipStream_t>(stream)};
    st = validate_prefill(a, false);
    if (st != DSA_OK) {
      std::string m = g_err;
      return fail(st, "layer %d: %s", l, m.c_str());
    }
  }
  for (int l = 0; l < N; ++l) {
    LayerRange range("indexcache prefill", l, pattern[l]);
    if (pattern[l] == 'F') {
      PrefillArgs a{q[l], q_scale ? q_scale[l] : nullptr, q_scale_head_stride, k[l],
                    k_scale ? k_scale[l] : nullptr, w[l], L, H, D, topk, dt, tcache, nullptr, nullptr,
                    workspace, workspace_bytes, static_cast<hipStream_t>(stream)};
      st = launch_prefill(a);
      if (st != DSA_OK) {
        std::string m = g_err;
        return fail(st, "layer %d: %s", l, m.c_str());
      }
    }
    if (hook) hook(l, src[l], tcache, stream, user);
  }
  if (src_layer_out) memcpy(src_layer_out, src.data(), sizeof(int32_t) * (size_t)N);
  return ok();
}

dsa_status indexcache_run_decode_layers(const char* pattern, int N, const uint16_t* const* q,
                                        const uint16_t* const* w, const uint8_t* const* k_cache,
                                        const float* const* k_scale, const int32_t* seq_lens, int B, int Lmax,
                                        int H, int D, int topk, int32_t* tcache, int32_t* src_layer_out,
                                        indexcache_layer_fn hook, void* user, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  std::vector<int32_t> src((size_t)(N > 0 ? N : 1));
  dsa_status st = indexcache_resolve(pattern, N, src.data());
  if (st != DSA_OK) return st;
  if (!q || !w || !k_cache || !k_scale)
    return fail(DSA_ERR_INVALID_ARG, "q, w, k_cache and k_scale pointer arrays must not be NULL");
  if (!tcache) return fail(DSA_ERR_INVALID_ARG, "tcache must not be NULL");
  auto args = [&](int l) {
    return DecodeArgs{q[l], w[l], k_cache[l], k_scale[l], seq_lens, B, Lmax, H, D, topk, tcache, nullptr,
                      workspace, workspace_bytes, static_cast<hipStream_t>(stream)};
  };
  // validate every F layer before enqueueing anything
  for (int l = 0; l < N; ++l) {
    if (pattern[l] != 'F') continue;
    st = validate_decode(args(l));
    if (st != DSA_OK) {
      std::string m = g_err;
      return fail(st, "layer %d: %s", l, m.c_str());
    }
  }
  for (int l = 0; l < N; ++l) {
    LayerRange range("indexcache decode", l, pattern[l]);
    if (pattern[l] == 'F') {
      st = launch_decode(args(l));
      if (st != DSA_OK) {
        std::string m = g_err;
        return fail(st, "layer %d: %s", l, m.c_str());
      }
    }
    if (hook) hook(l, src[l], tcache, stream, user);
  }
  if (src_layer_out) memcpy(src_layer_out, src.data(), sizeof(int32_t) * (size_t)N);
  return ok();
}

dsa_status indexcache_greedy_search(int N, int steps, indexcache_loss_fn loss, void* user, char* pattern_out,
                                    double* loss_trace, int32_t* flipped) {
  if (N < 1) return fail(DSA_ERR_INVALID_ARG, "N must be >= 1 (got %d)", N);
  if (steps < 0 || steps > N - 1) return fail(DSA_ERR_INVALID_ARG, "steps must be in [0, N-1] (got %d)", steps);
  if (!loss || !pattern_out) return fail(DSA_ERR_INVALID_ARG, "loss and pattern_out must not be NULL");
  std::string pat((size_t)N, 'F');
  double cur = loss(pat.c_str(), N, user);
  if (std::isnan(cur)) return fail(DSA_ERR_INVALID_ARG, "loss returned NaN for the all-F pattern");
  if (loss_trace) loss_trace[0] = cur;
  for (int step = 0; step < steps; ++step) {
    int best_l = -1;
    double best = 0.0;
    for (int l = 1; l < N; ++l) {   // the first layer stays F
      if (pat[(size_t)l] != 'F') continue;
      pat[(size_t)l] = 'S';
      const double v = loss(pat.c_str(), N, user);
      pat[(size_t)l] = 'F';
      if (std::isnan(v)) return fail(DSA_ERR_INVALID_ARG, "loss returned NaN at step %d, layer %d", step, l);
      if (best_l < 0 || v < best) {   // strict: the lowest layer wins a tie
        best_l = l;
        best = v;
      }
    }
    pat[(size_t)best_l] = 'S';
    if (loss_trace) loss_trace[step + 1] = best;
    if (flipped) flipped[step] = best_l;
  }
  memcpy(pattern_out, pat.c_str(), (size_t)N + 1);
  return ok();
}

dsa_status indexcache_overlap_proxy_loss(const char* pattern, int N, const double* ratio, double* loss) {
  if (!ratio || !loss) return fail(DSA_ERR_INVALID_ARG, "ratio and loss must not be NULL");
  std::vector<int32_t> src((size_t)(N > 0 ? N : 1));
  dsa_status st = indexcache_resolve(pattern, N, src.data());
  if (st != DSA_OK) return st;
  double lost = 0.0;
  for (int l = 0; l < N; ++l)
    if (pattern[l] == 'S') lost += 1.0 - ratio[(size_t)l * N + src[l]];
  *loss = lost / N;
  return ok();
}

dsa_status mli_resolve(const char* pattern, int N, int32_t* attn_src) {
  std::vector<int32_t> src((size_t)(N > 0 ? N : 1));
  dsa_status st = indexcache_resolve(pattern, N, src.data());
  if (st != DSA_OK) return st;
  int prev_f = -1;   // last F layer strictly before l
  for (int l = 0; l < N; ++l) {
    if (attn_src) attn_src[l] = prev_f >= 0 ? prev_f : l;
    if (pattern[l] == 'F') prev_f = l;
  }
  return ok();
}

dsa_status indexcache_run_decode_layers_mli(const char* pattern, int N, const uint16_t* const* q,
                                            const uint16_t* const* w, const uint8_t* const* k_cache,
                                            const float* const* k_scale, const int32_t* seq_lens, int B,
                                            int Lmax, int H, int D, int topk, int32_t* sel_buf,
                                            int32_t* attn_src_out, indexcache_layer_fn attn, void* user,
                                            void* workspace, size_t workspace_bytes, void* stream,
                                            void* side_stream) {
  std::vector<int32_t> asrc((size_t)(N > 0 ? N : 1));
  dsa_status st = mli_resolve(pattern, N, asrc.data());
  if (st != DSA_OK) return st;
  if (!q || !w || !k_cache || !k_scale)
    return fail(DSA_ERR_INVALID_ARG, "q, w, k_cache and k_scale pointer arrays must not be NULL");
  if (!sel_buf) return fail(DSA_ERR_INVALID_ARG, "sel_buf must not be NULL");
  hipStream_t main_s = static_cast<hipStream_t>(stream), side_s = static_cast<hipStream_t>(side_stream);
  const size_t slot = (size_t)(B > 0 ? B : 0) * (size_t)(topk > 0 ? topk : 0);
  // the i-th F layer writes slot i of sel_buf
  std::vector<int> slot_of((size_t)N, -1);
  for (int l = 0, nf = 0; l < N; ++l)
    if (pattern[l] == 'F') slot_of[l] = nf++;
  auto args = [&](int l) {
    return DecodeArgs{q[l], w[l], k_cache[l], k_scale[l], seq_lens, B, Lmax, H, D, topk,
                      sel_buf + (size_t)slot_of[l] * slot, nullptr, workspace, workspace_bytes, side_s};
  };
  for (int l = 0; l < N; ++l) {
    if (pattern[l] != 'F') continue;
    st = validate_decode(args(l));
    if (st != DSA_OK) {
      std::string m = g_err;
      return fail(st, "layer %d: %s", l, m.c_str());
    }
  }
  // Every F layer has a slot of its own, so the indexers never wait for the
  // attention: after the fork, the only cross-stream edges are "attention of
  // layer l waits for the indexer that wrote its selection" and the final
  // join.  Same-device streams need no system-scope fence.
  EventSet es;
  hipError_t e = es.create(4, hipEventDisableTiming | hipEventDisableSystemFence);
  if (e != hipSuccess) return hip_fail(e, "event create");
  hipEvent_t* written = es.ev;   // ring of two: slot i records written[i & 1]
  hipEvent_t ev_start = es.ev[2], ev_end = es.ev[3];
  if ((e = hipEventRecord(ev_start, main_s)) != hipSuccess || (e = hipStreamWaitEvent(side_s, ev_start, 0)) != hipSuccess)
    return hip_fail(e, "stream fork");
  int waited = -1;   // slot whose completion `stream` already waits for
  for (int l = 0; l < N; ++l) {
    LayerRange range("mli decode", l, pattern[l]);
    if (pattern[l] == 'F') {
      st = launch_decode(args(l));
      if (st != DSA_OK) {
        std::string m = g_err;
        return fail(st, "layer %d: %s", l, m.c_str());
      }
      if ((e = hipEventRecord(written[slot_of[l] & 1], side_s)) != hipSuccess) return hip_fail(e, "event record");
    }
    // written[i & 1] was last recorded by slot i: the attended slot is the
    // newest or the one before it
    const int sl = slot_of[asrc[l]];
    if (sl != waited) {
      if ((e = hipStreamWaitEvent(main_s, written[sl & 1], 0)) != hipSuccess) return hip_fail(e, "stream wait");
      waited = sl;
    }
    if (attn) attn(l, asrc[l], sel_buf + (size_t)sl * slot, stream, user);
  }
  // the main stream continues after the side stream's last work
  if ((e = hipEventRecord(ev_end, side_s)) != hipSuccess || (e = hipStreamWaitEvent(main_s, ev_end, 0)) != hipSuccess)
    return hip_fail(e, "stream join");
  if (attn_src_out) memcpy(attn_src_out, asrc.data(), sizeof(int32_t) * (size_t)N);
  return ok();
}

dsa_status standin_sparse_attention_workspace(int B, int topk, size_t* bytes) {
  if (!bytes) return fail(DSA_ERR_INVALID_ARG, "bytes must not be NULL");
  if (B < 1 || topk < 1 || topk > kMaxTopk) return fail(DSA_ERR_INVALID_ARG, "bad sizes B=%d topk=%d", B, topk);
  *bytes = (size_t)B * dsa::standin_attn_splits(topk) * dsa::STANDIN_PART * sizeof(float);
  return ok();
}

dsa_status standin_sparse_attention(const uint16_t* q, const uint16_t* latent, const int32_t* sel, int B, int Lmax,
                                    int topk, float scale, float* out, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  size_t need = 0;
  dsa_status st = standin_sparse_attention_workspace(B, topk, &need);
  if (st != DSA_OK) return st;
  if (Lmax < 1) return fail(DSA_ERR_INVALID_ARG, "Lmax must be >= 1");
  if (!q || !latent || !sel || !out) return fail(DSA_ERR_INVALID_ARG, "q, latent, sel and out must not be NULL");
  if (!aligned16(q) || !aligned16(latent) || !aligned16(out))
    return fail(DSA_ERR_INVALID_ARG, "q, latent and out must be 16-byte aligned");
  if (!workspace || workspace_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(DSA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  dsa::StandinAttnParams p{q, latent, sel, B, Lmax, topk, scale, static_cast<float*>(workspace), out};
  hipError_t e = dsa::standin_attn_launch(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "stand-in attention launch");
  return ok();
}

// ---------------------------------------------------------------------------

dsa_status topk_overlap_matrix(const int32_t* const* idx, int N, int L, int topk, int64_t row_begin,
                               int64_t row_end, int64_t row_stride, uint64_t* out_counts, double* out_ratio,
                               void* stream) {
  if (!idx || !out_counts) return fail(DSA_ERR_INVALID_ARG, "idx and out_counts must not be NULL");
  if (N < 1 || N > dsa::OVERLAP_MAX_N) return fail(DSA_ERR_INVALID_ARG, "N must be in [1, %d]", dsa::OVERLAP_MAX_N);
  if (L < 1 || topk < 1) return fail(DSA_ERR_INVALID_ARG, "L and topk must be >= 1");
  if (row_begin < 0 || row_end > L || row_begin >= row_end || row_stride < 1)
    return fail(DSA_ERR_INVALID_ARG, "rows must satisfy 0 <= row_begin < row_end <= L and row_stride >= 1");
  for (int i = 0; i < N; ++i)
    if (!idx[i]) return fail(DSA_ERR_INVALID_ARG, "idx[%d] is NULL", i);
  dsa::OverlapParams p{};
  for (int i = 0; i < N; ++i) p.idx[i] = idx[i];
  p.N = N;
  p.L = L;
  p.topk = topk;
  p.row_begin = row_begin;
  p.row_end = row_end;
  p.row_stride = row_stride;
  p.counts = reinterpret_cast<unsigned long long*>(out_counts);
  int cus = 0;
  if (device_cus(&cus) != 0) return fail(DSA_ERR_HIP, "no HIP device");
  const long long nrows = (row_end - row_begin + row_stride - 1) / row_stride;
  long long grid = (long long)dsa::overlap_blocks_per_cu(N) * cus;   // one pass of resident workgroups
  if (grid > nrows) grid = nrows;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = dsa::overlap_launch(p, (int)grid, s);
  if (e != hipSuccess) return hip_fail(e, "overlap launch");
  if (out_ratio) {
    std::vector<uint64_t> h((size_t)N * N);
    e = hipMemcpyAsync(h.data(), out_counts, h.size() * sizeof(uint64_t), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "overlap readback");
    const double den = (double)topk * (double)nrows;
    for (size_t i = 0; i < h.size(); ++i) out_ratio[i] = (double)h[i] / den;
  }
  return ok();
}

}  // extern "C"
