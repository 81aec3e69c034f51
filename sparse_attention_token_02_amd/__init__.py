"""Python binding of the gfx950 lightning-indexer library (``libdsa_indexer.so``).

Argument marshalling only: every function below takes torch tensors that
already live on the GPU, passes their device pointers and the current HIP
stream to the C entry point of the same name (declared in
``include/dsa_indexer.h``), and raises ``DsaError`` when it returns a
non-zero status.  Outputs and workspaces the caller does not pass are
allocated with torch.  There is no other implementation: importing this
package fails if the HIP library has not been built
(``python -m sparse_attention_token_02_amd.build``).
"""
from __future__ import annotations

import ctypes
import os

# torch ships its own HIP runtime.  Import it before loading the library so the
# library's libamdhip64.so.7 dependency resolves to that same, already-loaded
# runtime: two HIP runtimes in one process cannot share device pointers.
import torch  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa_indexer.so")

DSA_OK, DSA_ERR_INVALID_ARG, DSA_ERR_UNSUPPORTED, DSA_ERR_WORKSPACE, DSA_ERR_HIP = range(5)
DSA_BF16, DSA_FP8_E4M3 = 0, 1

EXPORTS = (
    "dsa_last_error", "dsa_abi_version",
    "dsa_indexer_topk_prefill_workspace", "dsa_indexer_topk_prefill", "dsa_indexer_topk_prefill_chunk",
    "dsa_indexer_topk_prefill_varlen_workspace", "dsa_indexer_topk_prefill_varlen",
    "dsa_indexer_topk_decode_workspace", "dsa_indexer_topk_decode", "dsa_indexer_topk_decode_noalloc",
    "dsa_indexer_topk_decode_paged",
    "indexcache_resolve", "indexcache_run_layers", "indexcache_run_decode_layers",
    "indexcache_greedy_search", "indexcache_overlap_proxy_loss", "mli_resolve",
    "indexcache_run_decode_layers_mli", "standin_sparse_attention_workspace", "standin_sparse_attention",
    "topk_overlap_matrix",
)

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m sparse_attention_token_02_amd.build`")

_lib = ctypes.CDLL(LIB_PATH)

_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
HOOK_T = ctypes.CFUNCTYPE(None, _i32, _i32, _vp, _vp, _vp)
LOSS_T = ctypes.CFUNCTYPE(ctypes.c_double, ctypes.c_char_p, _i32, _vp)

_lib.dsa_last_error.restype = ctypes.c_char_p
_lib.dsa_last_error.argtypes = []
_lib.dsa_abi_version.restype = _i32
_lib.dsa_abi_version.argtypes = []
_lib.dsa_indexer_topk_prefill_workspace.restype = _i32
_lib.dsa_indexer_topk_prefill_workspace.argtypes = [_i32, _i32, _i32, _i32, _i32, ctypes.POINTER(_sz)]
_lib.dsa_indexer_topk_prefill.restype = _i32
_lib.dsa_indexer_topk_prefill.argtypes = [_vp, _vp, _i64, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                          _vp, _vp, _vp, _vp, _sz, _vp]
_lib.dsa_indexer_topk_prefill_chunk.restype = _i32
_lib.dsa_indexer_topk_prefill_chunk.argtypes = [_vp, _vp, _i64, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                                _vp, _vp, _vp, _sz, _vp]
_lib.dsa_indexer_topk_prefill_varlen_workspace.restype = _i32
_lib.dsa_indexer_topk_prefill_varlen_workspace.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, ctypes.POINTER(_sz)]
_lib.dsa_indexer_topk_prefill_varlen.restype = _i32
_lib.dsa_indexer_topk_prefill_varlen.argtypes = [_vp, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                                 _i32, _i32, _vp, _vp, _vp, _sz, _vp]
_lib.dsa_indexer_topk_decode_workspace.restype = _i32
_lib.dsa_indexer_topk_decode_workspace.argtypes = [_i32, _i32, _i32, _i32, _i32, ctypes.POINTER(_sz)]
_lib.dsa_indexer_topk_decode.restype = _i32
_lib.dsa_indexer_topk_decode.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                         _vp, _vp, _vp, _sz, _vp]
_lib.dsa_indexer_topk_decode_noalloc.restype = _i32
_lib.dsa_indexer_topk_decode_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp]
_lib.dsa_indexer_topk_decode_paged.restype = _i32
_lib.dsa_indexer_topk_decode_paged.argtypes = [_vp, _vp, _vp, _vp, _i32, _i32, _vp, _i32, _vp, _i32, _i32, _i32, _i32,
                                               _vp, _vp, _vp, _sz, _vp]
_lib.indexcache_resolve.restype = _i32
_lib.indexcache_resolve.argtypes = [ctypes.c_char_p, _i32, ctypes.POINTER(ctypes.c_int32)]
_lib.indexcache_run_layers.restype = _i32
_lib.indexcache_run_layers.argtypes = [ctypes.c_char_p, _i32, ctypes.POINTER(_vp), ctypes.POINTER(_vp), _i64,
                                       ctypes.POINTER(_vp), ctypes.POINTER(_vp), ctypes.POINTER(_vp),
                                       _i32, _i32, _i32, _i32, _i32, _vp, ctypes.POINTER(ctypes.c_int32),
                                       HOOK_T, _vp, _vp, _sz, _vp]
_lib.indexcache_run_decode_layers.restype = _i32
_lib.indexcache_run_decode_layers.argtypes = [ctypes.c_char_p, _i32, ctypes.POINTER(_vp), ctypes.POINTER(_vp),
                                              ctypes.POINTER(_vp), ctypes.POINTER(_vp), _vp, _i32, _i32, _i32,
                                              _i32, _i32, _vp, ctypes.POINTER(ctypes.c_int32), HOOK_T, _vp, _vp,
                                              _sz, _vp]
_lib.indexcache_greedy_search.restype = _i32
_lib.indexcache_greedy_search.argtypes = [_i32, _i32, LOSS_T, _vp, ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                          ctypes.POINTER(ctypes.c_int32)]
_lib.indexcache_overlap_proxy_loss.restype = _i32
_lib.indexcache_overlap_proxy_loss.argtypes = [ctypes.c_char_p, _i32, ctypes.POINTER(ctypes.c_double),
                                               ctypes.POINTER(ctypes.c_double)]
_lib.mli_resolve.restype = _i32
_lib.mli_resolve.argtypes = [ctypes.c_char_p, _i32, ctypes.POINTER(ctypes.c_int32)]
_lib.indexcache_run_decode_layers_mli.restype = _i32
_lib.indexcache_run_decode_layers_mli.argtypes = [ctypes.c_char_p, _i32, ctypes.POINTER(_vp), ctypes.POINTER(_vp),
                                                  ctypes.POINTER(_vp), ctypes.POINTER(_vp), _vp, _i32, _i32, _i32,
                                                  _i32, _i32, _vp, ctypes.POINTER(ctypes.c_int32), HOOK_T, _vp,
                                                  _vp, _sz, _vp, _vp]
_lib.standin_sparse_attention_workspace.restype = _i32
_lib.standin_sparse_attention_workspace.argtypes = [_i32, _i32, ctypes.POINTER(_sz)]
_lib.standin_sparse_attention.restype = _i32
_lib.standin_sparse_attention.argtypes = [_vp, _vp, _vp, _i32, _i32, _i32, ctypes.c_float, _vp, _vp, _sz, _vp]
_lib.topk_overlap_matrix.restype = _i32
_lib.topk_overlap_matrix.argtypes = [ctypes.POINTER(_vp), _i32, _i32, _i32, _i64, _i64, _i64, _vp,
                                     ctypes.POINTER(ctypes.c_double), _vp]


class DsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"dsa status {status}: {message}")
        self.status = status


def _check(rc: int) -> None:
    if rc != DSA_OK:
        raise DsaError(rc, _lib.dsa_last_error().decode())


def lib() -> ctypes.CDLL:
    """The loaded shared library (for callers that want the raw C ABI)."""
    return _lib


def dsa_last_error() -> str:
    return _lib.dsa_last_error().decode()


def dsa_abi_version() -> int:
    return _lib.dsa_abi_version()


def _dt(dt) -> int:
    if dt in ("fp8", DSA_FP8_E4M3):
        return DSA_FP8_E4M3
    if dt in ("bf16", DSA_BF16):
        return DSA_BF16
    raise ValueError(f"unknown dtype {dt!r}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _record(tensors, device, *streams):
    """Tensors this binding allocated (on the current stream's pool) are used
    by kernels enqueued on ``streams``: tell torch's caching allocator, so that
    it does not hand their memory to other work before those kernels end."""
    import torch
    cur = torch.cuda.current_stream(device).cuda_stream
    for s in streams:
        if s is None:
            continue
        ts = torch.cuda.ExternalStream(s, device=device) if isinstance(s, int) else s
        if ts.cuda_stream == cur:
            continue
        for t in tensors:
            if t is not None:
                t.record_stream(ts)


def _workspace(nbytes: int, device, workspace, *streams):
    import torch
    if workspace is not None:
        return workspace
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)
    _record([ws], device, *streams)
    return ws


def _new(shape, dtype, device, stream):
    """An output allocated here, recorded on the stream its kernels run on."""
    import torch
    t = torch.empty(shape, dtype=dtype, device=device)
    _record([t], device, stream)
    return t


def dsa_indexer_topk_prefill_workspace(L: int, H: int, D: int, topk: int, dt) -> int:
    n = _sz(0)
    _check(_lib.dsa_indexer_topk_prefill_workspace(L, H, D, topk, _dt(dt), ctypes.byref(n)))
    return n.value


def dsa_indexer_topk_prefill(q, q_scale, k, k_scale, w, topk: int, dt, *, q_scale_head_stride: int = 0,
                             out_idx=None, out_topk_score=None, out_dense_score=None,
                             want_scores: bool = False, want_dense: bool = False,
                             workspace=None, stream=None):
    """q [L,H,D] (uint8 e4m3 codes or bf16), k [L,D], w [L,H] bf16, scales fp32 or None.
    Returns (idx [L,topk] int32, topk scores or None, dense scores or None)."""
    import torch
    L, H, D = q.shape
    dev = q.device
    if out_idx is None:
        out_idx = _new((L, topk), torch.int32, dev, stream)
    if out_topk_score is None and want_scores:
        out_topk_score = _new((L, topk), torch.float32, dev, stream)
    if out_dense_score is None and want_dense:
        out_dense_score = _new((L, L), torch.float32, dev, stream)
    ws = _workspace(dsa_indexer_topk_prefill_workspace(L, H, D, topk, dt), dev, workspace, stream)
    _check(_lib.dsa_indexer_topk_prefill(
        _ptr(q), _ptr(q_scale), q_scale_head_stride, _ptr(k), _ptr(k_scale), _ptr(w), L, H, D, topk, _dt(dt),
        _ptr(out_idx), _ptr(out_topk_score), _ptr(out_dense_score), _ptr(ws), ws.numel(), _stream(stream)))
    return out_idx, out_topk_score, out_dense_score


def dsa_indexer_topk_prefill_chunk(q, q_scale, k, k_scale, w, q_offset: int, topk: int, dt, *,
                                   q_scale_head_stride: int = 0, out_idx=None, out_topk_score=None,
                                   want_scores: bool = False, workspace=None, stream=None):
    """A block of query rows at positions q_offset .. q_offset+Lq-1: q [Lq,H,D],
    w [Lq,H], q_scale [Lq] or [Lq,H] or None; k [q_offset+Lq, D], k_scale
    [q_offset+Lq] or None.  Returns (idx [Lq,topk] int32, topk scores or None)."""
    import torch
    Lq, H, D = q.shape
    dev = q.device
    if k.shape[0] != q_offset + Lq:
        raise ValueError(f"k must hold q_offset + Lq = {q_offset + Lq} keys (has {k.shape[0]})")
    if out_idx is None:
        out_idx = _new((Lq, topk), torch.int32, dev, stream)
    if out_topk_score is None and want_scores:
        out_topk_score = _new((Lq, topk), torch.float32, dev, stream)
    ws = _workspace(dsa_indexer_topk_prefill_workspace(Lq, H, D, topk, dt), dev, workspace, stream)
    _check(_lib.dsa_indexer_topk_prefill_chunk(
        _ptr(q), _ptr(q_scale), q_scale_head_stride, _ptr(k), _ptr(k_scale), _ptr(w), q_offset, Lq, H, D, topk,
        _dt(dt), _ptr(out_idx), _ptr(out_topk_score), _ptr(ws), ws.numel(), _stream(stream)))
    return out_idx, out_topk_score


def dsa_indexer_topk_prefill_varlen_workspace(nseq: int, total_q: int, H: int, D: int, topk: int, dt) -> int:
    v = _sz(0)
    _check(_lib.dsa_indexer_topk_prefill_varlen_workspace(nseq, total_q, H, D, topk, _dt(dt), ctypes.byref(v)))
    return v.value


def dsa_indexer_topk_prefill_varlen(q, q_scale, k, k_scale, w, cu_seqlens_q, cu_seqlens_k, topk: int, dt, *,
                                    q_scale_head_stride: int = 0, out_idx=None, out_topk_score=None,
                                    want_scores: bool = False, workspace=None, stream=None):
    """Packed ragged batch in one launch: q [total_q,H,D], w [total_q,H],
    k [total_k,D]; cu_seqlens_* are device int32 tensors of nseq+1 entries.
    Returns (idx [total_q,topk], topk scores or None)."""
    import torch
    TQ, H, D = q.shape
    TK = k.shape[0]
    dev = q.device
    nseq = cu_seqlens_q.numel() - 1
    if cu_seqlens_k.numel() != nseq + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    if out_idx is None:
        out_idx = _new((TQ, topk), torch.int32, dev, stream)
    if out_topk_score is None and want_scores:
        out_topk_score = _new((TQ, topk), torch.float32, dev, stream)
    ws = _workspace(dsa_indexer_topk_prefill_varlen_workspace(nseq, TQ, H, D, topk, dt), dev, workspace, stream)
    _check(_lib.dsa_indexer_topk_prefill_varlen(
        _ptr(q), _ptr(q_scale), q_scale_head_stride, _ptr(k), _ptr(k_scale), _ptr(w), _ptr(cu_seqlens_q),
        _ptr(cu_seqlens_k), nseq, TQ, TK, H, D, topk, _dt(dt), _ptr(out_idx), _ptr(out_topk_score), _ptr(ws),
        ws.numel(), _stream(stream)))
    return out_idx, out_topk_score


def dsa_indexer_topk_decode_workspace(B: int, Lmax: int, H: int, D: int, topk: int) -> int:
    n = _sz(0)
    _check(_lib.dsa_indexer_topk_decode_workspace(B, Lmax, H, D, topk, ctypes.byref(n)))
    return n.value


def dsa_indexer_topk_decode(q, w, k_cache, k_scale, seq_lens, topk: int, *, out_idx=None,
                            out_topk_score=None, want_scores: bool = False, workspace=None, stream=None):
    """q [B,H,D] bf16, w [B,H] bf16, k_cache [B,Lmax,D] e4m3 codes, k_scale [B,Lmax] fp32,
    seq_lens [B] int32 (device).  Returns (idx [B,topk] int32, scores or None)."""
    import torch
    B, H, D = q.shape
    Lmax = k_cache.shape[1]
    dev = q.device
    if out_idx is None:
        out_idx = _new((B, topk), torch.int32, dev, stream)
    if out_topk_score is None and want_scores:
        out_topk_score = _new((B, topk), torch.float32, dev, stream)
    ws = _workspace(dsa_indexer_topk_decode_workspace(B, Lmax, H, D, topk), dev, workspace, stream)
    _check(_lib.dsa_indexer_topk_decode(
        _ptr(q), _ptr(w), _ptr(k_cache), _ptr(k_scale), _ptr(seq_lens), B, Lmax, H, D, topk,
        _ptr(out_idx), _ptr(out_topk_score), _ptr(ws), ws.numel(), _stream(stream)))
    return out_idx, out_topk_score


def dsa_indexer_topk_decode_noalloc(q, w, k_cache, k_scale, seq_lens, topk: int, out_idx, out_topk_score=None,
                                    stream=None):
    """dsa_indexer_topk_decode into caller-provided outputs (out_idx [B,topk]
    int32, out_topk_score [B,topk] fp32 or None) with the library's
    per-device scratch: nothing is allocated, here or in the library."""
    B, H, D = q.shape
    Lmax = k_cache.shape[1]
    _check(_lib.dsa_indexer_topk_decode_noalloc(
        _ptr(q), _ptr(w), _ptr(k_cache), _ptr(k_scale), _ptr(seq_lens), B, Lmax, H, D, topk,
        _ptr(out_idx), _ptr(out_topk_score), _stream(stream)))
    return out_idx, out_topk_score


def dsa_indexer_topk_decode_paged(q, w, k_pages, k_scale_pages, block_table, seq_lens, topk: int, *, out_idx=None,
                                  out_topk_score=None, want_scores: bool = False, workspace=None, stream=None):
    """q [B,H,D] bf16, w [B,H] bf16, k_pages [P,page,D] e4m3 codes, k_scale_pages
    [P,page] fp32, block_table [B,max_blocks] int32, seq_lens [B] int32 (device).
    Returns (idx [B,topk] int32, scores or None)."""
    import torch
    B, H, D = q.shape
    num_pages, page = k_pages.shape[0], k_pages.shape[1]
    max_blocks = block_table.shape[1]
    dev = q.device
    if out_idx is None:
        out_idx = _new((B, topk), torch.int32, dev, stream)
    if out_topk_score is None and want_scores:
        out_topk_score = _new((B, topk), torch.float32, dev, stream)
    ws = _workspace(dsa_indexer_topk_decode_workspace(B, max_blocks * page, H, D, topk), dev, workspace, stream)
    _check(_lib.dsa_indexer_topk_decode_paged(
        _ptr(q), _ptr(w), _ptr(k_pages), _ptr(k_scale_pages), num_pages, page, _ptr(block_table), max_blocks,
        _ptr(seq_lens), B, H, D, topk, _ptr(out_idx), _ptr(out_topk_score), _ptr(ws), ws.numel(), _stream(stream)))
    return out_idx, out_topk_score


def indexcache_resolve(pattern: str) -> list[int]:
    N = len(pattern)
    src = (ctypes.c_int32 * max(N, 1))()
    _check(_lib.indexcache_resolve(pattern.encode(), N, src))
    return list(src[:N])


def _ptr_array(ts):
    arr = (_vp * len(ts))()
    for i, t in enumerate(ts):
        arr[i] = _ptr(t) if t is not None else None
    return arr


def indexcache_run_layers(pattern: str, q, q_scale, k, k_scale, w, topk: int, dt, *,
                          q_scale_head_stride: int = 0, tcache=None, hook=None, workspace=None, stream=None):
    """Per-layer lists of device tensors (entries of S layers may be None).
    ``hook(layer, src_layer, tcache)`` runs after every layer, on the host, in
    order (work it enqueues on the current stream is ordered with the schedule).
    Returns (tcache, src_layer list)."""
    import torch
    N = len(pattern)
    f0 = next(i for i, c in enumerate(pattern) if c == "F") if "F" in pattern else 0
    L, H, D = q[f0].shape
    dev = q[f0].device
    if tcache is None:
        tcache = _new((L, topk), torch.int32, dev, stream)
    ws = _workspace(dsa_indexer_topk_prefill_workspace(L, H, D, topk, dt), dev, workspace, stream)
    src = (ctypes.c_int32 * max(N, 1))()
    errors = []

    def _hook(layer, src_layer, idx_ptr, stream_ptr, user):
        try:
            hook(layer, src_layer, tcache)
        except Exception as e:  # surfaced after the call returns
            errors.append(e)

    cb = HOOK_T(_hook) if hook is not None else HOOK_T()
    _check(_lib.indexcache_run_layers(
        pattern.encode(), N, _ptr_array(q), _ptr_array(q_scale) if q_scale is not None else None,
        q_scale_head_stride, _ptr_array(k), _ptr_array(k_scale) if k_scale is not None else None,
        _ptr_array(w), L, H, D, topk, _dt(dt), _ptr(tcache), src, cb, None, _ptr(ws), ws.numel(),
        _stream(stream)))
    if errors:
        raise errors[0]
    return tcache, list(src[:N])


def indexcache_run_decode_layers(pattern: str, q, w, k_cache, k_scale, seq_lens, topk: int, *, tcache=None,
                                 hook=None, workspace=None, stream=None):
    """One decode step through the F/S schedule.  q, w, k_cache, k_scale are
    per-layer lists of device tensors with the shapes of
    ``dsa_indexer_topk_decode`` (entries of S layers may be None); seq_lens
    [B] int32 is shared by all layers.  ``hook(layer, src_layer, tcache)`` as
    in ``indexcache_run_layers``.  Returns (tcache [B,topk], src_layer list)."""
    import torch
    N = len(pattern)
    f0 = next(i for i, c in enumerate(pattern) if c == "F") if "F" in pattern else 0
    B, H, D = q[f0].shape
    Lmax = k_cache[f0].shape[1]
    dev = q[f0].device
    if tcache is None:
        tcache = _new((B, topk), torch.int32, dev, stream)
    ws = _workspace(dsa_indexer_topk_decode_workspace(B, Lmax, H, D, topk), dev, workspace, stream)
    src = (ctypes.c_int32 * max(N, 1))()
    errors = []

    def _hook(layer, src_layer, idx_ptr, stream_ptr, user):
        try:
            hook(layer, src_layer, tcache)
        except Exception as e:  # surfaced after the call returns
            errors.append(e)

    cb = HOOK_T(_hook) if hook is not None else HOOK_T()
    _check(_lib.indexcache_run_decode_layers(
        pattern.encode(), N, _ptr_array(q), _ptr_array(w), _ptr_array(k_cache), _ptr_array(k_scale),
        _ptr(seq_lens), B, Lmax, H, D, topk, _ptr(tcache), src, cb, None, _ptr(ws), ws.numel(),
        _stream(stream)))
    if errors:
        raise errors[0]
    return tcache, list(src[:N])


def indexcache_greedy_search(N: int, steps: int, loss):
    """Greedy F/S search from all F: ``loss(pattern: str) -> float`` is called
    for the all-F pattern and for every trial.  Returns (pattern, loss trace
    [steps + 1], flipped layer per step)."""
    import math
    out = ctypes.create_string_buffer(N + 1)
    trace = (ctypes.c_double * (steps + 1))()
    flipped = (ctypes.c_int32 * max(steps, 1))()
    errors = []

    def _loss(pat, n, user):
        try:
            return float(loss(pat.decode()))
        except Exception as e:  # surfaced after the call returns
            errors.append(e)
            return math.nan

    rc = _lib.indexcache_greedy_search(N, steps, LOSS_T(_loss), None, out, trace, flipped)
    if errors:
        raise errors[0]
    _check(rc)
    return out.value.decode(), list(trace), list(flipped[:steps])


def indexcache_overlap_proxy_loss(pattern: str, ratio) -> float:
    """Overlap-proxy loss of a pattern (a labelled baseline), ratio: [N, N]
    host float64 overlap ratios of an all-F run."""
    import numpy as np
    r = np.ascontiguousarray(ratio, dtype=np.float64)
    v = ctypes.c_double(0.0)
    _check(_lib.indexcache_overlap_proxy_loss(pattern.encode(), len(pattern),
                                              r.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), ctypes.byref(v)))
    return v.value


def mli_resolve(pattern: str) -> list[int]:
    N = len(pattern)
    src = (ctypes.c_int32 * max(N, 1))()
    _check(_lib.mli_resolve(pattern.encode(), N, src))
    return list(src[:N])


def indexcache_run_decode_layers_mli(pattern: str, q, w, k_cache, k_scale, seq_lens, topk: int, *, sel_buf=None,
                                     attn=None, workspace=None, stream=None, side_stream=None):
    """One decode step through the lagged (multi-layer indexer) schedule.
    Per-layer lists as in ``indexcache_run_decode_layers``.  ``attn(layer,
    src_layer, selection)`` runs on the host for every layer, in order, with
    ``selection`` the [B, topk] slot of ``sel_buf`` that layer attends; work it
    enqueues on ``stream`` (the current stream by default) is ordered after
    that selection is written.  ``side_stream`` (a torch stream) runs the
    indexers.  Returns (sel_buf [F, B, topk], slot i = the i-th F layer's
    selection, attn_src list)."""
    import torch
    N = len(pattern)
    f0 = next(i for i, c in enumerate(pattern) if c == "F") if "F" in pattern else 0
    B, H, D = q[f0].shape
    Lmax = k_cache[f0].shape[1]
    dev = q[f0].device
    nf = pattern.count("F")
    if sel_buf is None:
        sel_buf = torch.empty((max(nf, 1), B, topk), dtype=torch.int32, device=dev)
        sel_alloc = True
    else:
        sel_alloc = False
    if sel_buf.shape[0] < nf or tuple(sel_buf.shape[1:]) != (B, topk) or not sel_buf.is_contiguous():
        raise ValueError(f"sel_buf must be a contiguous [{nf}+, {B}, {topk}] int32 tensor")
    if side_stream is None:
        side_stream = torch.cuda.Stream(device=dev)
    ws = _workspace(dsa_indexer_topk_decode_workspace(B, Lmax, H, D, topk), dev, workspace, stream, side_stream)
    if sel_alloc:   # written on the side stream, read on `stream`
        _record([sel_buf], dev, stream, side_stream)
    src = (ctypes.c_int32 * max(N, 1))()
    slots = {sel_buf[i].data_ptr(): sel_buf[i] for i in range(sel_buf.shape[0])}
    errors = []

    def _hook(layer, src_layer, idx_ptr, stream_ptr, user):
        try:
            attn(layer, src_layer, slots[idx_ptr])
        except Exception as e:  # surfaced after the call returns
            errors.append(e)

    cb = HOOK_T(_hook) if attn is not None else HOOK_T()
    _check(_lib.indexcache_run_decode_layers_mli(
        pattern.encode(), N, _ptr_array(q), _ptr_array(w), _ptr_array(k_cache), _ptr_array(k_scale),
        _ptr(seq_lens), B, Lmax, H, D, topk, _ptr(sel_buf), src, cb, None, _ptr(ws), ws.numel(),
        _stream(stream), _stream(side_stream)))
    if errors:
        raise errors[0]
    return sel_buf, list(src[:N])


def standin_sparse_attention_workspace(B: int, topk: int) -> int:
    n = _sz(0)
    _check(_lib.standin_sparse_attention_workspace(B, topk, ctypes.byref(n)))
    return n.value


def standin_sparse_attention(q, latent, sel, scale: float, *, out=None, workspace=None, stream=None):
    """q [B,576] bf16, latent [B,Lmax,576] bf16, sel [B,topk] int32 (device).
    Returns out [B,512] fp32."""
    import torch
    B = q.shape[0]
    Lmax = latent.shape[1]
    topk = sel.shape[1]
    if out is None:
        out = _new((B, 512), torch.float32, q.device, stream)
    ws = _workspace(standin_sparse_attention_workspace(B, topk), q.device, workspace, stream)
    _check(_lib.standin_sparse_attention(_ptr(q), _ptr(latent), _ptr(sel), B, Lmax, topk, float(scale), _ptr(out),
                                         _ptr(ws), ws.numel(), _stream(stream)))
    return out


def topk_overlap_matrix(idx, topk: int, *, row_begin=None, row_end=None, row_stride: int = 1,
                        out_counts=None, ratio: bool = True, stream=None):
    """idx: list of N device int32 tensors [L, topk].  Returns (counts [N,N] uint64
    device tensor, ratio numpy [N,N] or None).  Default rows: topk-1 .. L-1."""
    import numpy as np
    import torch
    N = len(idx)
    L = idx[0].shape[0]
    rb = topk - 1 if row_begin is None else row_begin
    re_ = L if row_end is None else row_end
    if out_counts is None:
        out_counts = _new((N, N), torch.uint64, idx[0].device, stream)
    r = np.empty((N, N), dtype=np.float64) if ratio else None
    rp = r.ctypes.data_as(ctypes.POINTER(ctypes.c_double)) if ratio else None
    _check(_lib.topk_overlap_matrix(_ptr_array(idx), N, L, topk, rb, re_, row_stride, _ptr(out_counts), rp,
                                    _stream(stream)))
    return out_counts, r
