/*
 * dsa_indexer.h -- C ABI of the gfx950 (MI355X) lightning-indexer library.
 *
 * The library computes the DeepSeek Sparse Attention lightning indexer, its
 * per-query top-k selection, the IndexCache Full/Shared layer schedule that
 * reuses the selected indices, and the cross-layer overlap statistic.
 *
 * Sources (web pages, cited by title and section):
 *  [IC]  "IndexCache deep-dive report" (zako-mio.github.io, IndexShare 03):
 *        abstract and section 1.1 -- the indexer is a multi-head ReLU-gated
 *        dot product run in FP8 that scores all earlier tokens and keeps the
 *        top k = 2048; section 1.2 -- overlap |T_i ∩ T_j| / k; section 2.1 --
 *        F layers run the indexer and write the index cache, S layers reuse
 *        the nearest earlier F layer's indices, the first layer is always F.
 *  [BA]  "IndexCache" news article (hub.baai.ac.cn/view/53293), figure on the
 *        inference loop -- the cache is one temporary index tensor that every
 *        F layer overwrites, with no memory beyond what DSA already holds.
 *  [IS]  "Index Share logic" tech note (foosynaptic.github.io), sections 2 and
 *        4.2 -- per layer: indexer, top-k, sparse attention; an S layer takes
 *        cached_indices = the last F layer's indices.
 *  [ML]  "Multi-layer Indexer" abstract (equalang.com) -- at decode the
 *        indexer scores the whole cache and keeps the k = 2048 best.
 *
 * The score of query t against key s is
 *     score(t, s) = k_scale[s] * sum_h w[t,h] * q_scale[t,h] * ReLU(q[t,h] . k[s])
 * with one key vector per token shared by all heads (the pages print no
 * equation; this is the multi-head ReLU-gated dot product of [IC] 1.1).
 * The selection keeps the min(k, n) best keys under the total order "score
 * descending, then key index ascending" (ties go to the lower index) and
 * returns them in ascending key order, padded with -1 (score -inf).
 *
 * Conventions for every entry point:
 *  - All tensors are caller-owned device memory, row-major and contiguous.
 *    The library allocates nothing and keeps no state between calls except a
 *    thread-local error string.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *    stream) unless stated otherwise.  Arguments are validated on the host
 *    before anything is enqueued; on an error nothing is enqueued and the
 *    status says why (dsa_last_error() has the message).
 *  - e4m3 is the OCP 8-bit float E4M3 ("e4m3fn": bias 7, max 448, no inf,
 *    S.1111.111 = NaN); bf16 is the top half of an IEEE float32.  Inputs must
 *    be finite.
 *  - q, k and the decode cache must be 16-byte aligned.
 *  - Identical inputs give identical output bytes (deterministic).
 */
#ifndef DSA_INDEXER_H
#define DSA_INDEXER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dsa_status {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = 1,   /* null pointer, bad size, misaligned pointer, bad pattern */
  DSA_ERR_UNSUPPORTED = 2,   /* shape the kernels are not built for */
  DSA_ERR_WORKSPACE = 3,     /* workspace missing or smaller than the query says */
  DSA_ERR_HIP = 4            /* a HIP call failed; the message has the HIP error */
} dsa_status;

typedef enum dsa_dtype {
  DSA_BF16 = 0,
  DSA_FP8_E4M3 = 1
} dsa_dtype;

/* Message of the last error on the calling thread ("" if none). */
const char* dsa_last_error(void);

/* ABI revision of this header (bumped on any signature change). */
int dsa_abi_version(void);

/* ------------------------------------------------------------------------
 * Prefill: one sequence of L tokens, causal, query t scores keys 0..t
 * (diagonal included).  [IC] abstract and 1.1.
 * ------------------------------------------------------------------------ */

/* Workspace bytes dsa_indexer_topk_prefill needs for these sizes on the
 * current HIP device. */
dsa_status dsa_indexer_topk_prefill_workspace(int L, int H, int D, int topk, dsa_dtype dt,
                                              size_t* bytes);

/*
 * q        [L, H, D] dt          query heads (e4m3 codes or bf16)
 * q_scale  fp32 or NULL (= 1)    element (t, h) at q_scale[t*(stride? H:1) + h*stride]:
 *                                q_scale_head_stride 0 = one scale per token ([L]),
 *                                1 = one per (token, head) ([L, H])
 * k        [L, D] dt             keys, one vector per token shared by all heads
 * k_scale  [L] fp32 or NULL (= 1)
 * w        [L, H] bf16           head weights
 * L >= 1; H a multiple of 8 with 8 <= H <= 128 (kernels are built for H in
 * {8, 16, 32, 64, 128}; other counts run on the next of these with zero
 * heads appended); D in {64, 128}; 1 <= topk <= 4096.
 * out_idx        [L, topk] int32  selected keys, ascending, -1 padded (written in full).
 *                A key whose score is NaN or -inf (finite but extreme inputs can
 *                overflow) is never selected; its row then holds fewer than
 *                min(topk, t+1) keys and is padded, still written in full.
 *                When neither scores nor dense scores are requested, rows with
 *                t + 1 <= topk may be answered without scoring them: every key
 *                0 .. t is then selected, whatever its score (with finite scores,
 *                the same selection).
 * out_topk_score [L, topk] fp32   scores aligned with out_idx, -inf padded; NULL to skip
 * out_dense_score [L, L] fp32     every score, -inf above the diagonal; NULL to skip;
 *                                 only for L <= 16384 (a debugging aid: the normal path
 *                                 never stores the L x L matrix)
 * workspace      device bytes, at least what the query above returns; its
 *                contents on entry do not matter.
 * Outputs must not alias inputs.
 */
dsa_status dsa_indexer_topk_prefill(const void* q, const float* q_scale, int64_t q_scale_head_stride,
                                    const void* k, const float* k_scale, const uint16_t* w,
                                    int L, int H, int D, int topk, dsa_dtype dt,
                                    int32_t* out_idx, float* out_topk_score, float* out_dense_score,
                                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Chunked prefill: a block of Lq query rows at absolute positions
 * q_offset .. q_offset + Lq - 1 of one sequence, against that sequence's
 * keys 0 .. q_offset + Lq - 1 (the keys of earlier chunks already in the
 * cache, then the chunk's own).  Row i of the block scores keys
 * 0 .. q_offset + i, as row q_offset + i of a whole-sequence prefill would,
 * and gets the same selection ([IS] 2: the indexer and top-k run per layer
 * over everything before the query; serving engines feed long prompts in
 * such chunks).
 * q [Lq, H, D], q_scale ([Lq] or [Lq, H]), w [Lq, H]: the block's rows;
 * k [q_offset + Lq, D], k_scale [q_offset + Lq]: all keys so far;
 * out_idx / out_topk_score [Lq, topk].  q_offset >= 0, Lq >= 1; other
 * arguments and limits as for dsa_indexer_topk_prefill (no dense output).
 * The workspace is dsa_indexer_topk_prefill_workspace(Lq, H, D, topk, dt).
 */
dsa_status dsa_indexer_topk_prefill_chunk(const void* q, const float* q_scale, int64_t q_scale_head_stride,
                                          const void* k, const float* k_scale, const uint16_t* w,
                                          int q_offset, int Lq, int H, int D, int topk, dsa_dtype dt,
                                          int32_t* out_idx, float* out_topk_score,
                                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Ragged batch of sequences, packed, in one launch: sequence i has the query
 * rows cu_seqlens_q[i] .. cu_seqlens_q[i+1]-1 and the keys
 * cu_seqlens_k[i] .. cu_seqlens_k[i+1]-1, its queries being the last
 * Lq_i = cu_seqlens_q[i+1] - cu_seqlens_q[i] of its Lk_i keys (a chunk as in
 * dsa_indexer_topk_prefill_chunk, q_offset = Lk_i - Lq_i; Lq_i = Lk_i is a
 * whole sequence, Lq_i = 0 contributes nothing).
 * cu_seqlens_q, cu_seqlens_k  DEVICE int32 [nseq + 1], read on the device:
 *            a sequence whose bounds are not 0 <= cu_q[i] <= cu_q[i+1] <=
 *            total_q, 0 <= cu_k[i] <= cu_k[i+1] <= total_k, Lq_i <= Lk_i is
 *            skipped (its rows are not written); nothing is read or written
 *            outside the arrays below whatever they hold.
 * q [total_q, H, D], q_scale ([total_q] or [total_q, H]), w [total_q, H],
 * out_idx / out_topk_score [total_q, topk]; k [total_k, D], k_scale [total_k].
 * Each row gets the selection of its own sequence, exactly as a call per
 * sequence would.  A one-workgroup kernel builds the work-item table on the
 * device (sequences longest first when nseq <= 1024, each sequence's
 * longest items first); one persistent launch then takes items from it.
 * Other arguments and limits as for dsa_indexer_topk_prefill.
 */
dsa_status dsa_indexer_topk_prefill_varlen_workspace(int nseq, int total_q, int H, int D, int topk, dsa_dtype dt,
                                                     size_t* bytes);
dsa_status dsa_indexer_topk_prefill_varlen(const void* q, const float* q_scale, int64_t q_scale_head_stride,
                                           const void* k, const float* k_scale, const uint16_t* w,
                                           const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int nseq,
                                           int total_q, int total_k, int H, int D, int topk, dsa_dtype dt,
                                           int32_t* out_idx, float* out_topk_score,
                                           void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Decode: B sequences with one new query each, at position len_b - 1, whose
 * own key is already in the cache; the query scores the whole cache
 * (keys 0 .. len_b - 1).  [ML] abstract; [IS] section 2 (the indexer runs
 * per layer at every decode step).
 * ------------------------------------------------------------------------ */

dsa_status dsa_indexer_topk_decode_workspace(int B, int Lmax, int H, int D, int topk, size_t* bytes);

/*
 * q        [B, H, D] bf16        one query per sequence
 * w        [B, H] bf16           head weights
 * k_cache  [B, Lmax, D] e4m3     indexer key cache
 * k_scale  [B, Lmax] fp32        one scale per cached token
 * seq_lens [B] int32, device     1 <= len_b <= Lmax (read on the device only, so
 *                                not checked: a value outside [0, Lmax] is clamped
 *                                into it, and a length of 0 gives a row of -1 with
 *                                -inf scores)
 * B >= 1; H a multiple of 8 with 8 <= H <= 128 (run on the kernel built for
 * the next of {16, 32, 64, 128}, zero heads appended); D in {64, 128};
 * 1 <= Lmax <= 262144; 1 <= topk <= 4096.
 * out_idx        [B, topk] int32 ascending, -1 padded
 * out_topk_score [B, topk] fp32 or NULL
 */
dsa_status dsa_indexer_topk_decode(const uint16_t* q, const uint16_t* w, const uint8_t* k_cache,
                                   const float* k_scale, const int32_t* seq_lens,
                                   int B, int Lmax, int H, int D, int topk,
                                   int32_t* out_idx, float* out_topk_score,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * dsa_indexer_topk_decode without a workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  The call allocates nothing: its
 * scratch is a 48 MiB array in device memory that the library holds on each
 * device from its load until the process ends, one copy per device, shared
 * by every call of this entry point on that device.  Calls that overlap in
 * time on one device race on it (serialise them, e.g. on one stream); a
 * call needs nothing cleared and leaves its contents behind.  Sizes whose
 * workspace (dsa_indexer_topk_decode_workspace) exceeds 48 MiB are rejected
 * with DSA_ERR_UNSUPPORTED before anything is enqueued; B = 32 sequences of
 * Lmax = 131072 fit.  Arguments, outputs and results as for
 * dsa_indexer_topk_decode.
 */
dsa_status dsa_indexer_topk_decode_noalloc(const uint16_t* q, const uint16_t* w, const uint8_t* k_cache,
                                           const float* k_scale, const int32_t* seq_lens,
                                           int B, int Lmax, int H, int D, int topk,
                                           int32_t* out_idx, float* out_topk_score, void* stream);

/*
 * Decode over a paged key cache, as serving engines keep it ([IS] 2: the
 * decode indexer scores each sequence's whole cache every step): the same
 * selection as dsa_indexer_topk_decode on the cache the pages describe.
 * k_pages       [num_pages, page_size, D] e4m3
 * k_scale_pages [num_pages, page_size] fp32
 * block_table   [B, max_blocks] int32, device: token s of sequence b is row
 *               s % page_size of page block_table[b, s / page_size]
 * page_size     a power of two >= 32; 1 <= max_blocks; the largest sequence
 *               is max_blocks * page_size <= 262144 tokens.
 * Entries for the blocks below ceil(len_b / page_size) must be page ids in
 * [0, num_pages); others are not read.  (An id outside the range is clamped
 * into it, so no access leaves the page arrays; the selection of that
 * sequence is then unspecified.)  q, w, seq_lens, outputs and limits as for
 * dsa_indexer_topk_decode; the workspace is
 * dsa_indexer_topk_decode_workspace(B, max_blocks * page_size, H, D, topk).
 */
dsa_status dsa_indexer_topk_decode_paged(const uint16_t* q, const uint16_t* w, const uint8_t* k_pages,
                                         const float* k_scale_pages, int num_pages, int page_size,
                                         const int32_t* block_table, int max_blocks,
                                         const int32_t* seq_lens, int B, int H, int D, int topk,
                                         int32_t* out_idx, float* out_topk_score,
                                         void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * IndexCache Full/Shared schedule.  [IC] 2.1, [BA] inference-loop figure,
 * [IS] 4.2.
 * ------------------------------------------------------------------------ */

/* Host only, no device work.  pattern: N characters from {F, S}, first one F
 * ([IC] 2.1: the first layer is always F).  src_layer (host [N], may be NULL)
 * receives src[l] = l for F and the nearest earlier F layer for S. */
dsa_status indexcache_resolve(const char* pattern, int N, int32_t* src_layer);

/* Called once per layer, in order, after that layer's indices are in
 * `idx` (for an S layer: the buffer the source F layer wrote, same pointer).
 * Work the hook enqueues on `stream` is ordered with the schedule. */
typedef void (*indexcache_layer_fn)(int layer, int src_layer, const int32_t* idx, void* stream,
                                    void* user);

/*
 * Runs the schedule over N layers of one prefill: an F layer runs
 * dsa_indexer_topk_prefill with its own inputs into `tcache`; an S layer
 * enqueues nothing and reuses `tcache` in place.
 * q, q_scale, k, k_scale, w: host arrays of N device pointers (entries of S
 * layers are not read and may be NULL; q_scale/k_scale arrays may be NULL).
 * tcache [L, topk] int32, caller-owned, overwritten at every F layer.
 * src_layer_out host [N] or NULL.  hook may be NULL.
 * The workspace is the prefill workspace for (L, H, D, topk, dt).
 */
dsa_status indexcache_run_layers(const char* pattern, int N,
                                 const void* const* q, const float* const* q_scale,
                                 int64_t q_scale_head_stride,
                                 const void* const* k, const float* const* k_scale,
                                 const uint16_t* const* w,
                                 int L, int H, int D, int topk, dsa_dtype dt,
                                 int32_t* tcache, int32_t* src_layer_out,
                                 indexcache_layer_fn hook, void* user,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * The same schedule for one decode step ([IS] 2: at decode every layer runs
 * its indexer at every step; [IC] 4.2: the decode-throughput gain comes from
 * the S layers skipping it).  An F layer runs dsa_indexer_topk_decode with its
 * own q, w and key cache into `tcache`; an S layer enqueues nothing and
 * reuses `tcache` in place.
 * q, w, k_cache, k_scale: host arrays of N device pointers with the shapes of
 *            dsa_indexer_topk_decode (entries of S layers are not read and may
 *            be NULL).
 * seq_lens   [B] int32, device, shared by every layer (one step of B
 *            sequences).
 * tcache     [B, topk] int32, caller-owned, overwritten at every F layer.
 * src_layer_out host [N] or NULL.  hook may be NULL; it runs after every
 * layer as in indexcache_run_layers.
 * The workspace is the decode workspace for (B, Lmax, H, D, topk).  Every F
 * layer is validated before anything is enqueued.
 */
dsa_status indexcache_run_decode_layers(const char* pattern, int N,
                                        const uint16_t* const* q, const uint16_t* const* w,
                                        const uint8_t* const* k_cache, const float* const* k_scale,
                                        const int32_t* seq_lens, int B, int Lmax, int H, int D, int topk,
                                        int32_t* tcache, int32_t* src_layer_out,
                                        indexcache_layer_fn hook, void* user,
                                        void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Training-free pattern search.  [IC] 3.1 (greedy layer selection): start
 * from all F; at every step try turning each remaining F layer into S,
 * score each trial with a calibration loss and commit the lowest; K steps
 * (K = 3N/4 for retention 1/4).  [IC] 5.2: a full run costs N(N-1)/2
 * evaluations, and similarity proxies do not predict the loss.
 * ------------------------------------------------------------------------ */

/* Loss of a pattern (N characters, NUL-terminated), e.g. a model's LM loss on
 * calibration data; the caller owns what it runs.  NaN is an error. */
typedef double (*indexcache_loss_fn)(const char* pattern, int N, void* user);

/*
 * Host only, no device work (the loss may do any).  Runs `steps` greedy
 * steps from all F (0 <= steps <= N-1; the first layer is never turned into
 * S).  Among trials with equal loss the lowest layer wins.
 * pattern_out  host char[N + 1]: the final pattern, NUL-terminated
 * loss_trace   host double[steps + 1] or NULL: the all-F loss, then the loss
 *              committed at every step
 * flipped      host int32[steps] or NULL: the layer turned into S at every step
 * The loss is called 1 + sum_{i<steps} (N-1-i) times, in layer order within
 * a step.
 */
dsa_status indexcache_greedy_search(int N, int steps, indexcache_loss_fn loss, void* user,
                                    char* pattern_out, double* loss_trace, int32_t* flipped);

/*
 * A similarity proxy for the loss, as a labelled baseline only ([IC] 5.2
 * reports that such proxies fail): the mean over all N layers of
 * 1 - ratio[l][src(l)] over the S layers, with ratio the N x N host overlap
 * ratio matrix of an all-F run (topk_overlap_matrix) and src the pattern's
 * source layers.  Host only.
 */
dsa_status indexcache_overlap_proxy_loss(const char* pattern, int N, const double* ratio, double* loss);

/* ------------------------------------------------------------------------
 * Multi-layer Indexer (lagged) decode schedule.  [ML] abstract: adjacent
 * layers select nearly the same tokens, so a layer attends the selection of
 * the previous indexer layer instead of its own; its own indexer then runs
 * concurrently with its attention.  Composed with F/S: S layers have no
 * indexer and attend the nearest earlier F layer's selection, as before.
 * ------------------------------------------------------------------------ */

/* Host only, no device work.  attn_src (host [N], may be NULL) receives the
 * layer whose selection layer l attends: the last F layer strictly before l,
 * or l itself when there is none (the first layer).  The pattern rules are
 * those of indexcache_resolve. */
dsa_status mli_resolve(const char* pattern, int N, int32_t* attn_src);

/*
 * One decode step through the lagged schedule, on two streams.  F layers run
 * dsa_indexer_topk_decode (inputs as in indexcache_run_decode_layers) on
 * `side_stream`, the i-th F layer into slot i of sel_buf; for every layer l,
 * in order, `attn(l, attn_src[l], selection, stream, user)` is called on the
 * host and enqueues that layer's attention on `stream` (the main one).
 * Ordering, by events (device scope, no system fence):
 *  - the side stream starts after the work already queued on `stream`;
 *  - layer l's attention waits for the indexer that wrote its selection;
 *  - on return, `stream` waits for the side stream's last work.
 * Every F layer has a slot of its own, so the indexers never wait for the
 * attention: each one overlaps the attention of the layers before it (and
 * whatever the caller enqueues on `stream` in between), and the whole step
 * is ordered on `stream`.
 * sel_buf        [F, B, topk] int32, caller-owned, F = number of F layers in
 *                the pattern; after the step slot i holds the i-th F layer's
 *                selection.  The `selection` pointer handed to attn is one
 *                slot.
 * attn_src_out   host [N] or NULL; attn may be NULL.
 * side_stream    another hipStream_t of the same device (the same stream as
 *                `stream`, or both NULL, gives a correct but serial schedule).
 * Every F layer is validated before anything is enqueued.  Four events are
 * created per call and released on return.
 */
dsa_status indexcache_run_decode_layers_mli(const char* pattern, int N,
                                            const uint16_t* const* q, const uint16_t* const* w,
                                            const uint8_t* const* k_cache, const float* const* k_scale,
                                            const int32_t* seq_lens, int B, int Lmax, int H, int D, int topk,
                                            int32_t* sel_buf, int32_t* attn_src_out,
                                            indexcache_layer_fn attn, void* user,
                                            void* workspace, size_t workspace_bytes,
                                            void* stream, void* side_stream);

/*
 * Stand-in consumer of a decode selection for the schedules above: one head
 * of sparse softmax attention per sequence over the selected rows of a bf16
 * latent cache (576 values per row, the first 512 of which are the value),
 * with the memory traffic of sparse MLA decode ([ML] abstract: each layer
 * attends only the k selected tokens).  It is not a model's attention layer.
 *   s_j = scale * q[b] . latent[b, T_j, 0:576]
 *   out[b] = sum_j softmax(s)_j latent[b, T_j, 0:512]
 * over the entries 0 <= T_j < Lmax of sel[b] (others, such as -1 padding,
 * are skipped; a row with none gives zeros).
 * q [B, 576] bf16, latent [B, Lmax, 576] bf16, sel [B, topk] int32,
 * out [B, 512] fp32, all device, q/latent/out 16-byte aligned.
 */
dsa_status standin_sparse_attention_workspace(int B, int topk, size_t* bytes);
dsa_status standin_sparse_attention(const uint16_t* q, const uint16_t* latent, const int32_t* sel,
                                    int B, int Lmax, int topk, float scale, float* out,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Cross-layer overlap.  [IC] 1.2.
 * ------------------------------------------------------------------------ */

/*
 * idx        host array of N device pointers, each [L, topk] int32, ascending
 *            non-negative indices then -1 padding (the selection outputs above:
 *            prefill rows, whose keys are <= t, or decode rows, one per
 *            sequence, whose keys run up to len_b - 1).  Keys above 2^30 - 1
 *            are not counted.
 * rows       t = row_begin, row_begin + row_stride, ... < row_end
 *            (0 <= row_begin < row_end <= L, row_stride >= 1)
 * out_counts [N, N] uint64, device: C[i][j] = sum over rows of |T_i(t) ∩ T_j(t)|
 * out_ratio  [N, N] fp64, host, or NULL: C / (topk * number of rows).  When it
 *            is given the call waits for the stream (synchronous).
 * 1 <= N <= 64.
 */
dsa_status topk_overlap_matrix(const int32_t* const* idx, int N, int L, int topk,
                               int64_t row_begin, int64_t row_end, int64_t row_stride,
                               uint64_t* out_counts, double* out_ratio, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_INDEXER_H */
