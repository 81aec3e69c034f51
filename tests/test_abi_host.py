"""C-ABI checks that need no GPU: the library loads, exports every function
declared in include/dsa_indexer.h, and rejects bad arguments on the host
before anything reaches HIP (no compute call is made here)."""
import ctypes
import os
import re

import pytest

import sparse_attention_token_02_amd as dsa
from synth import gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa_indexer.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^(?:dsa_status|const char\*|int)\s+(\w+)\s*\(", text, flags=re.M)
    return names


def test_header_declares_the_boundary():
    names = set(_declared())
    for n in ("dsa_indexer_topk_prefill", "dsa_indexer_topk_decode", "indexcache_run_layers",
              "topk_overlap_matrix"):
        assert n in names


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(dsa.LIB_PATH)
    names = _declared()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(dsa.EXPORTS)


def test_abi_version():
    assert dsa.dsa_abi_version() == 1


@pytest.mark.parametrize("name", ["all_F", "uniform_1_4", "searched_1_4"])
def test_resolve_matches_schedule_rule(name):
    p = gen.FS_PATTERNS[name]
    src = dsa.indexcache_resolve(p)
    for l, c in enumerate(p):
        assert src[l] == (l if c == "F" else max(j for j in range(l) if p[j] == "F"))
    assert sum(1 for l in range(47) if src[l] == l) == p.count("F")


@pytest.mark.parametrize("bad", ["SFF", "FXS", "F S", "f"])
def test_resolve_rejects(bad):
    with pytest.raises(dsa.DsaError) as e:
        dsa.indexcache_resolve(bad)
    assert e.value.status == dsa.DSA_ERR_INVALID_ARG


def test_resolve_length_mismatch_and_null():
    lib = dsa.lib()
    src = (ctypes.c_int32 * 4)()
    assert lib.indexcache_resolve(b"FSF", 4, src) == dsa.DSA_ERR_INVALID_ARG
    assert "length" in dsa.dsa_last_error()
    assert lib.indexcache_resolve(None, 3, src) == dsa.DSA_ERR_INVALID_ARG
    assert lib.indexcache_resolve(b"FSF", 3, None) == dsa.DSA_OK


def test_prefill_workspace_query():
    n = dsa.dsa_indexer_topk_prefill_workspace(32768, 64, 128, 2048, "fp8")
    assert n > 0
    small = dsa.dsa_indexer_topk_prefill_workspace(2048, 8, 64, 128, "bf16")
    assert 0 < small < n
    for args, st in [((0, 64, 128, 2048, "fp8"), dsa.DSA_ERR_INVALID_ARG),
                     ((1024, 64, 128, 0, "fp8"), dsa.DSA_ERR_INVALID_ARG),
                     ((1024, 64, 128, 5000, "fp8"), dsa.DSA_ERR_INVALID_ARG),
                     ((1024, 44, 128, 64, "fp8"), dsa.DSA_ERR_UNSUPPORTED),
                     ((1024, 136, 128, 64, "fp8"), dsa.DSA_ERR_UNSUPPORTED),
                     ((1024, 48, 32, 64, "bf16"), dsa.DSA_ERR_UNSUPPORTED),
                     ((1024, 64, 96, 64, "fp8"), dsa.DSA_ERR_UNSUPPORTED),
                     ((1024, 256, 128, 64, "fp8"), dsa.DSA_ERR_UNSUPPORTED)]:
        with pytest.raises(dsa.DsaError) as e:
            dsa.dsa_indexer_topk_prefill_workspace(*args)
        assert e.value.status == st, args
    # a head count between the built widths takes the next width's layout
    assert dsa.dsa_indexer_topk_prefill_workspace(1024, 48, 128, 64, "fp8") == \
        dsa.dsa_indexer_topk_prefill_workspace(1024, 64, 128, 64, "fp8")
    assert dsa.dsa_indexer_topk_prefill_workspace(1024, 24, 64, 64, "bf16") == \
        dsa.dsa_indexer_topk_prefill_workspace(1024, 32, 64, 64, "bf16")
    assert dsa.dsa_indexer_topk_prefill_workspace(1024, 72, 128, 64, "fp8") == \
        dsa.dsa_indexer_topk_prefill_workspace(1024, 128, 128, 64, "fp8")
    # the one-wave-per-SIMD configurations are built too
    for H, D, dt in [(128, 128, "fp8"), (128, 64, "fp8"), (128, 128, "bf16"), (128, 64, "bf16"), (64, 128, "bf16")]:
        assert dsa.dsa_indexer_topk_prefill_workspace(1024, H, D, 64, dt) > 0
    lib = dsa.lib()
    assert lib.dsa_indexer_topk_prefill_workspace(16, 8, 64, 4, 7, ctypes.byref(ctypes.c_size_t())) == \
        dsa.DSA_ERR_INVALID_ARG


FAKE = 1 << 20   # an aligned non-null address; never dereferenced (validation fails first)


def _prefill(lib, **kw):
    a = dict(q=FAKE, qs=None, qsh=0, k=FAKE, ks=None, w=FAKE, L=64, H=8, D=64, topk=8, dt=dsa.DSA_BF16,
             oi=FAKE, osc=None, od=None, ws=FAKE, wsb=1 << 30, stream=None)
    a.update(kw)
    return lib.dsa_indexer_topk_prefill(a["q"], a["qs"], a["qsh"], a["k"], a["ks"], a["w"], a["L"], a["H"],
                                        a["D"], a["topk"], a["dt"], a["oi"], a["osc"], a["od"], a["ws"],
                                        a["wsb"], a["stream"])


def test_prefill_rejects_before_any_device_call():
    lib = dsa.lib()
    assert _prefill(lib, q=None) == dsa.DSA_ERR_INVALID_ARG
    assert _prefill(lib, oi=None) == dsa.DSA_ERR_INVALID_ARG
    assert _prefill(lib, q=FAKE + 4) == dsa.DSA_ERR_INVALID_ARG            # misaligned
    assert _prefill(lib, qsh=2) == dsa.DSA_ERR_INVALID_ARG
    assert _prefill(lib, topk=0) == dsa.DSA_ERR_INVALID_ARG
    assert _prefill(lib, H=12) == dsa.DSA_ERR_UNSUPPORTED
    assert _prefill(lib, wsb=16) == dsa.DSA_ERR_WORKSPACE
    assert "workspace" in dsa.dsa_last_error()
    assert _prefill(lib, ws=None) == dsa.DSA_ERR_WORKSPACE
    assert _prefill(lib, L=20000, od=FAKE) == dsa.DSA_ERR_INVALID_ARG    # dense output limited


def test_prefill_chunk_rejects_before_any_device_call():
    lib = dsa.lib()

    def call(q0=100, lq=50, H=64, D=128, topk=16, ws=FAKE, wsb=1 << 30, oi=FAKE):
        return lib.dsa_indexer_topk_prefill_chunk(FAKE, None, 0, FAKE, None, FAKE, q0, lq, H, D, topk,
                                                  dsa.DSA_FP8_E4M3, oi, None, ws, wsb, None)
    assert call(q0=-1) == dsa.DSA_ERR_INVALID_ARG
    assert call(lq=0) == dsa.DSA_ERR_INVALID_ARG
    assert call(q0=2**31 - 10, lq=20) == dsa.DSA_ERR_INVALID_ARG
    assert call(oi=None) == dsa.DSA_ERR_INVALID_ARG
    assert call(wsb=16) == dsa.DSA_ERR_WORKSPACE
    assert call(H=12) == dsa.DSA_ERR_UNSUPPORTED


def test_prefill_varlen_rejects_before_any_device_call():
    lib = dsa.lib()

    def call(n=3, tq=30, tk=40, H=64, wsb=1 << 30, cq=FAKE, q=FAKE):
        return lib.dsa_indexer_topk_prefill_varlen(q, None, 0, FAKE, None, FAKE, cq, FAKE, n, tq, tk, H, 128, 16,
                                                   dsa.DSA_FP8_E4M3, FAKE, None, FAKE, wsb, None)
    assert call(n=0) == dsa.DSA_ERR_INVALID_ARG
    assert call(tq=-1) == dsa.DSA_ERR_INVALID_ARG
    assert call(tk=-1) == dsa.DSA_ERR_INVALID_ARG
    assert call(cq=None) == dsa.DSA_ERR_INVALID_ARG
    assert call(q=None) == dsa.DSA_ERR_INVALID_ARG
    assert call(H=12) == dsa.DSA_ERR_UNSUPPORTED
    assert call(wsb=16) == dsa.DSA_ERR_WORKSPACE
    assert call(tq=0) == dsa.DSA_OK                    # nothing to select: nothing enqueued
    n1 = dsa.dsa_indexer_topk_prefill_varlen_workspace(3, 30, 64, 128, 16, "fp8")
    n2 = dsa.dsa_indexer_topk_prefill_varlen_workspace(3, 3000, 64, 128, 16, "fp8")
    assert n2 > n1 > 0


def test_decode_rejects_before_any_device_call():
    lib = dsa.lib()
    n = dsa.dsa_indexer_topk_decode_workspace(32, 131072, 64, 128, 2048)
    assert n >= 32 * 131072 * 4

    def call(**kw):
        a = dict(q=FAKE, w=FAKE, c=FAKE, ks=FAKE, lens=FAKE, B=2, Lmax=1024, H=64, D=128, topk=16, oi=FAKE,
                 osc=None, ws=FAKE, wsb=1 << 30)
        a.update(kw)
        return lib.dsa_indexer_topk_decode(a["q"], a["w"], a["c"], a["ks"], a["lens"], a["B"], a["Lmax"], a["H"],
                                           a["D"], a["topk"], a["oi"], a["osc"], a["ws"], a["wsb"], None)
    assert call(lens=None) == dsa.DSA_ERR_INVALID_ARG
    assert call(B=0) == dsa.DSA_ERR_INVALID_ARG
    assert call(H=12) == dsa.DSA_ERR_UNSUPPORTED
    assert call(H=136) == dsa.DSA_ERR_UNSUPPORTED
    assert call(Lmax=1 << 20) == dsa.DSA_ERR_UNSUPPORTED
    assert call(wsb=100) == dsa.DSA_ERR_WORKSPACE
    assert call(c=FAKE + 8) == dsa.DSA_ERR_INVALID_ARG


def test_decode_paged_rejects_before_any_device_call():
    lib = dsa.lib()

    def call(page=64, npages=10, table=FAKE, mb=16, H=64, wsb=1 << 30, c=FAKE):
        return lib.dsa_indexer_topk_decode_paged(FAKE, FAKE, c, FAKE, npages, page, table, mb, FAKE, 2, H, 128, 16,
                                                 FAKE, None, FAKE, wsb, None)
    assert call(page=48) == dsa.DSA_ERR_INVALID_ARG
    assert call(page=16) == dsa.DSA_ERR_INVALID_ARG
    assert call(npages=0) == dsa.DSA_ERR_INVALID_ARG
    assert call(table=None) == dsa.DSA_ERR_INVALID_ARG
    assert call(mb=8193) == dsa.DSA_ERR_UNSUPPORTED          # more than 262144 tokens
    assert call(H=12) == dsa.DSA_ERR_UNSUPPORTED
    assert call(H=136) == dsa.DSA_ERR_UNSUPPORTED
    assert call(wsb=64) == dsa.DSA_ERR_WORKSPACE
    assert call(c=FAKE + 4) == dsa.DSA_ERR_INVALID_ARG


def test_overlap_rejects_before_any_device_call():
    lib = dsa.lib()
    arr = (ctypes.c_void_p * 2)(FAKE, FAKE)

    def call(N=2, L=100, topk=8, rb=7, re_=100, rs=1, counts=FAKE, idx=arr):
        return lib.topk_overlap_matrix(idx, N, L, topk, rb, re_, rs, counts, None, None)
    assert call(N=0) == dsa.DSA_ERR_INVALID_ARG
    assert call(N=65) == dsa.DSA_ERR_INVALID_ARG
    assert call(rb=50, re_=50) == dsa.DSA_ERR_INVALID_ARG
    assert call(re_=101) == dsa.DSA_ERR_INVALID_ARG
    assert call(rs=0) == dsa.DSA_ERR_INVALID_ARG
    assert call(counts=None) == dsa.DSA_ERR_INVALID_ARG
    bad = (ctypes.c_void_p * 2)(FAKE, None)
    assert call(idx=bad) == dsa.DSA_ERR_INVALID_ARG


def test_run_layers_rejects_before_any_device_call():
    lib = dsa.lib()
    P = ctypes.c_void_p * 3
    q, k, w = P(FAKE, FAKE, FAKE), P(FAKE, FAKE, FAKE), P(FAKE, FAKE, FAKE)
    hook = dsa.HOOK_T()

    def call(pattern=b"FSF", N=3, tc=FAKE, wsb=1 << 30, qq=q):
        return lib.indexcache_run_layers(pattern, N, qq, None, 0, k, None, w, 64, 8, 64, 8, dsa.DSA_BF16, tc,
                                         None, hook, None, FAKE, wsb, None)
    assert call(pattern=b"SFF") == dsa.DSA_ERR_INVALID_ARG
    assert call(N=4) == dsa.DSA_ERR_INVALID_ARG
    assert call(tc=None) == dsa.DSA_ERR_INVALID_ARG
    assert call(wsb=16) == dsa.DSA_ERR_WORKSPACE
    assert "layer 0" in dsa.dsa_last_error()
    q_bad = P(FAKE, FAKE, None)      # layer 2 is F and has no q
    assert call(qq=q_bad) == dsa.DSA_ERR_INVALID_ARG
    assert "layer 2" in dsa.dsa_last_error()
    q_s_null = P(FAKE, None, FAKE)   # S layer entries are not read
    assert call(qq=q_s_null, wsb=16) == dsa.DSA_ERR_WORKSPACE


def test_run_decode_layers_rejects_before_any_device_call():
    lib = dsa.lib()
    P = ctypes.c_void_p * 3
    arr = lambda *v: P(*v)
    full = arr(FAKE, FAKE, FAKE)
    hook = dsa.HOOK_T()

    def call(pattern=b"FSF", N=3, tc=FAKE, wsb=1 << 30, qq=full, H=64, cache=full):
        return lib.indexcache_run_decode_layers(pattern, N, qq, full, cache, full, FAKE, 2, 1024, H, 128, 16, tc,
                                                None, hook, None, FAKE, wsb, None)
    assert call(pattern=b"SFF") == dsa.DSA_ERR_INVALID_ARG
    assert call(pattern=b"FXF") == dsa.DSA_ERR_INVALID_ARG
    assert call(N=2) == dsa.DSA_ERR_INVALID_ARG
    assert call(tc=None) == dsa.DSA_ERR_INVALID_ARG
    assert call(wsb=16) == dsa.DSA_ERR_WORKSPACE
    assert "layer 0" in dsa.dsa_last_error()
    assert call(H=12) == dsa.DSA_ERR_UNSUPPORTED
    assert call(H=136) == dsa.DSA_ERR_UNSUPPORTED
    assert call(qq=arr(FAKE, FAKE, None)) == dsa.DSA_ERR_INVALID_ARG     # layer 2 is F and has no q
    assert "layer 2" in dsa.dsa_last_error()
    assert call(cache=arr(FAKE, FAKE, FAKE + 8)) == dsa.DSA_ERR_INVALID_ARG   # misaligned cache of layer 2
    assert call(qq=arr(FAKE, None, FAKE), cache=arr(FAKE, None, FAKE), wsb=16) == dsa.DSA_ERR_WORKSPACE


@pytest.mark.parametrize("name", sorted(gen.FS_PATTERNS))
def test_mli_resolve_matches_schedule_rule(name):
    import oracle
    pat = gen.FS_PATTERNS[name]
    assert dsa.mli_resolve(pat) == oracle.mli_resolve(pat)
    assert dsa.mli_resolve("FSFFS") == [0, 0, 0, 2, 3]
    with pytest.raises(dsa.DsaError):
        dsa.mli_resolve("SFF")


def test_run_decode_layers_mli_rejects_before_any_device_call():
    lib = dsa.lib()
    P = ctypes.c_void_p * 3
    full = P(FAKE, FAKE, FAKE)
    hook = dsa.HOOK_T()

    def call(pattern=b"FSF", N=3, sb=FAKE, wsb=1 << 30, qq=full, H=64):
        return lib.indexcache_run_decode_layers_mli(pattern, N, qq, full, full, full, FAKE, 2, 1024, H, 128, 16,
                                                    sb, None, hook, None, FAKE, wsb, None, None)
    assert call(pattern=b"SFF") == dsa.DSA_ERR_INVALID_ARG
    assert call(sb=None) == dsa.DSA_ERR_INVALID_ARG
    assert call(wsb=16) == dsa.DSA_ERR_WORKSPACE
    assert "layer 0" in dsa.dsa_last_error()
    assert call(H=12) == dsa.DSA_ERR_UNSUPPORTED
    assert call(H=136) == dsa.DSA_ERR_UNSUPPORTED
    assert call(qq=P(FAKE, FAKE, None)) == dsa.DSA_ERR_INVALID_ARG
    assert "layer 2" in dsa.dsa_last_error()


def test_standin_attention_rejects_before_any_device_call():
    lib = dsa.lib()
    n = dsa.standin_sparse_attention_workspace(32, 2048)
    assert n == 32 * 16 * (4 + 512) * 4

    def call(q=FAKE, lat=FAKE, sel=FAKE, B=2, Lmax=100, topk=16, out=FAKE, ws=FAKE, wsb=1 << 20):
        return lib.standin_sparse_attention(q, lat, sel, B, Lmax, topk, 0.5, out, ws, wsb, None)
    assert call(sel=None) == dsa.DSA_ERR_INVALID_ARG
    assert call(B=0) == dsa.DSA_ERR_INVALID_ARG
    assert call(topk=5000) == dsa.DSA_ERR_INVALID_ARG
    assert call(Lmax=0) == dsa.DSA_ERR_INVALID_ARG
    assert call(lat=FAKE + 2) == dsa.DSA_ERR_INVALID_ARG
    assert call(wsb=64) == dsa.DSA_ERR_WORKSPACE


def test_greedy_search_matches_oracle():
    """The library's search against the oracle's, on seeded table losses
    (a hash of the pattern) and on the overlap proxy of a random matrix."""
    import hashlib
    import numpy as np
    import oracle
    for N, steps in [(1, 0), (2, 1), (9, 6), (20, 15)]:
        loss = lambda p: int(hashlib.sha256(p.encode()).hexdigest()[:6], 16) / 2.0 ** 24
        assert dsa.indexcache_greedy_search(N, steps, loss) == oracle.fs_greedy_search(N, steps, loss)
    rng = np.random.default_rng(2)
    R = rng.random((12, 12))
    R = (R + R.T) / 2
    np.fill_diagonal(R, 1.0)
    for p in ["F" * 12, "FSFSFSFSFSFS", "FSSSSSSSSSSF"]:
        assert dsa.indexcache_overlap_proxy_loss(p, R) == pytest.approx(oracle.overlap_proxy_loss(p, R), abs=1e-15)
    proxy = lambda p: dsa.indexcache_overlap_proxy_loss(p, R)
    assert dsa.indexcache_greedy_search(12, 9, proxy) == oracle.fs_greedy_search(12, 9, proxy)


def test_greedy_search_rejects_and_reports_loss_errors():
    with pytest.raises(dsa.DsaError):
        dsa.indexcache_greedy_search(5, 5, lambda p: 0.0)
    with pytest.raises(dsa.DsaError):
        dsa.indexcache_greedy_search(0, 0, lambda p: 0.0)
    with pytest.raises(dsa.DsaError):
        dsa.indexcache_greedy_search(4, 2, lambda p: float("nan"))

    class Boom(Exception):
        pass

    def bad(p):
        raise Boom(p)
    with pytest.raises(Boom):
        dsa.indexcache_greedy_search(4, 2, bad)
    with pytest.raises(dsa.DsaError):
        dsa.indexcache_overlap_proxy_loss("SFF", [[1.0] * 3] * 3)


def test_one_hip_runtime_in_process():
    """The library binds to the HIP runtime torch loaded (never a second copy)."""
    import torch  # noqa: F401
    maps = open("/proc/self/maps").read().splitlines()
    paths = {l.split()[-1] for l in maps if "libamdhip64" in l}
    assert len(paths) == 1, paths


def test_peak_library_exports_its_header():
    """The measured-peak library used by the benchmark exports every function
    include/dsa_peak.h declares (no kernel is launched here)."""
    from sparse_attention_token_02_amd import peak
    text = open(os.path.join(ROOT, "include", "dsa_peak.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^int\s+(\w+)\s*\(", text, flags=re.M)
    lib = ctypes.CDLL(peak.LIB_PATH)
    assert set(names) == set(peak.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_noalloc_decode_refuses_sizes_beyond_its_scratch_on_the_host():
    lib = dsa.lib()
    rc = lib.dsa_indexer_topk_decode_noalloc(None, None, None, None, None, 64, 131072, 64, 128, 2048, None, None,
                                             None)
    assert rc == dsa.DSA_ERR_UNSUPPORTED
    assert b"allocation-free" in lib.dsa_last_error()
