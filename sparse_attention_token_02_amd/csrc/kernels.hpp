// Internal interface between the C-ABI layer (abi.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dsa_indexer.h"

namespace dsa {

constexpr int OVERLAP_MAX_N = 64;

struct PrefillParams {
  const uint8_t* q;          // [L - q0, H, D] e4m3 codes or bf16 (as bytes)
  const float* q_scale;      // nullable; element (t, h) at t*qs_row + h*qs_head
  int64_t qs_row;
  int64_t qs_head;
  const uint8_t* k;          // [L, D]
  const float* k_scale;      // [L], nullable
  const uint16_t* w;         // [L, H] bf16
  int hr;                    // H of the caller's q / q_scale / w (the kernel's width pads it)
  int L;                     // keys (query rows are the absolute positions q0 .. L-1)
  int q0;                    // absolute position of query row 0 (0 for a whole sequence)
  int topk;
  int cap;                   // candidate list capacity per row
  int sample_m;              // keys per row in the threshold sample (0: no sample)
  int32_t* out_idx;          // [L - q0, topk]
  float* out_score;          // [L - q0, topk], nullable
  float* out_dense;          // [L - q0, L], nullable
  float* ws_sc;              // [grid, rows_per_item, cap]
  int32_t* ws_ix;            // [grid, rows_per_item, cap]
  int* counter;              // work counter
  int n_items;               // ceil((L - q0) / rows_per_item)
  // Ragged batch (items != null): item i reads its sequence from items[i] =
  // {q row of position 0 (q row of position t is t + x), first key row, key
  // count, first query position of the item}, *n_items_dev items in all; L,
  // q0 and n_items above are then unused.
  const int4* items;
  const int* n_items_dev;
};

// Builds the ragged-batch item table from device cu_seqlens (one workgroup):
// sequences whose bounds are not 0 <= cu_q[i] <= cu_q[i+1] <= total_q,
// 0 <= cu_k[i] <= cu_k[i+1] <= total_k, Lq <= Lk are skipped; the longest
// key range goes first (by sequence, when nseq <= 1024), and within a
// sequence its longest item first.  Also clears the work counter.
hipError_t prefill_varlen_prepare(const int32_t* cu_q, const int32_t* cu_k, int nseq, int total_q, int total_k,
                                  int rows_per_item, int4* items, int* n_items, int* counter, hipStream_t stream);

constexpr int MAX_TOPK = 4096;   // the largest k the library accepts

// Head counts: any multiple of 8 up to 128 runs on the kernels built for the
// next width in {8, 16, 32, 64, 128} (decode: {16, 32, 64, 128}), the extra
// heads zero (their dot products, weights and scores contribute nothing).
inline int prefill_head_width(int H) {
  if (H < 8 || H > 128 || H % 8) return 0;
  return H <= 8 ? 8 : H <= 16 ? 16 : H <= 32 ? 32 : H <= 64 ? 64 : 128;
}
inline int decode_head_width(int H) {
  if (H < 8 || H > 128 || H % 8) return 0;
  return H <= 16 ? 16 : H <= 32 ? 32 : H <= 64 ? 64 : 128;
}

// Per-sequence header of the decode workspace: the pool claim counter
// (count in the low half, the owning call's tag in the high half) and the
// generation word that every call's select advances.
struct DecodeHdr {
  unsigned long long pool;
  uint32_t gen;
  uint32_t pad;
};

struct DecodeParams {
  const uint16_t* q;         // [B, hr, D] bf16
  const uint16_t* w;         // [B, hr] bf16
  int hr;                    // the caller's H (the kernel's width pads it with zero heads)
  const uint8_t* cache;      // [B, Lmax, D] e4m3
  const float* k_scale;      // [B, Lmax]
  const int32_t* lens;       // [B] device
  int B;
  int Lmax;
  int topk;
  int32_t* out_idx;          // [B, topk]
  float* out_score;          // [B, topk], nullable
  DecodeHdr* hdr;            // workspace [B]
  uint32_t nonce;            // per launch, from the host
  uint32_t* hist;            // workspace [B, nwg, PW]: per-workgroup 16-bit histograms
  int2* wgcut;               // workspace [B, nwg]: per list (lowest bin kept, entries)
  uint2* cand;               // workspace [B, nwg, keys per workgroup]: (key, index) lists
  // paged cache (block_table != null): cache = pages [num_pages, 2^page_shift, D],
  // k_scale = [num_pages, 2^page_shift]; token s of sequence b lives in page
  // block_table[b * max_blocks + (s >> page_shift)]; Lmax = max_blocks << page_shift
  const int32_t* block_table;
  int max_blocks;
  int page_shift;
  int num_pages;
};

// per sequence: score workgroups, histogram words, list entries
struct DecodeWsSizes {
  size_t nwg, hist_words, cand_entries;
};

// Stand-in sparse attention (one head): latent rows of STANDIN_DK bf16 values,
// the first STANDIN_DV of which are the value vector.
constexpr int STANDIN_DK = 576;
constexpr int STANDIN_DV = 512;
constexpr int STANDIN_ROWS = 128;             // selection entries per workgroup
constexpr int STANDIN_PART = 4 + STANDIN_DV;  // floats per partial: max, sum, pad, weighted rows

struct StandinAttnParams {
  const uint16_t* q;         // [B, STANDIN_DK] bf16
  const uint16_t* latent;    // [B, Lmax, STANDIN_DK] bf16
  const int32_t* sel;        // [B, topk], -1 padded
  int B;
  int Lmax;
  int topk;
  float scale;
  float* part;               // workspace [B, splits, STANDIN_PART]
  float* out;                // [B, STANDIN_DV] fp32
};

int standin_attn_splits(int topk);
hipError_t standin_attn_launch(const StandinAttnParams& p, hipStream_t stream);

// Largest key index the overlap kernel counts; larger entries are ignored.
constexpr int OVERLAP_MAX_KEY = (1 << 30) - 1;

struct OverlapParams {
  const int32_t* idx[OVERLAP_MAX_N];   // N device pointers, each [L, topk]
  int N;
  int L;
  int topk;
  long long row_begin;
  long long row_end;
  long long row_stride;
  unsigned long long* counts;          // [N, N] device
};

// prefill.hip
bool prefill_supported(int dt, int H, int D);
int prefill_rows_per_item(int dt, int H, int D);
int prefill_list_capacity(int dt, int H, int D, int topk);
int prefill_sample_keys(int dt, int H, int D);
hipError_t prefill_launch(const PrefillParams& p, int dt, int H, int D, int grid, hipStream_t stream);

// decode.hip
bool decode_supported(int H, int D, int Lmax);
size_t decode_select_lds_bytes(int Lmax, int topk);
DecodeWsSizes decode_ws_sizes(int Lmax);
hipError_t decode_launch(const DecodeParams& p, int H, int D, hipStream_t stream);
// the allocation-free entry point's per-device scratch: its size, and the
// current device's address
size_t decode_scratch_bytes();
hipError_t decode_scratch(void** ptr);

// overlap.hip
size_t overlap_lds_bytes(int N);
int overlap_blocks_per_cu(int N);
hipError_t overlap_launch(const OverlapParams& p, int grid, hipStream_t stream);

}  // namespace dsa
