"""Host-only checks of the C ABI: every declared symbol is exported, and the
argument validation rejects bad calls before anything reaches the GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def csa():
    import compressed_sparse_long_compress_amd as m

    return m


def declared_functions():
    src = open(os.path.join(ROOT, "include", "csa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M)))


def test_every_declared_symbol_is_exported(csa):
    names = declared_functions()
    assert {"csa_compress", "csa_index_scores", "csa_topk", "csa_sparse_mqa", "hca_dense_mqa"} <= set(names)
    lib = ctypes.CDLL(csa.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/csa.h but not exported"
    assert set(names) == set(csa.EXPORTS)


def test_version(csa):
    hdr = open(os.path.join(ROOT, "include", "csa.h")).read()
    v = int(re.search(r"#define CSA_VERSION (\d+)", hdr).group(1))
    assert csa.version() == v


def _kv(csa, cap=16):
    return csa._Kv(None, None, None, cap)


def test_compress_validation(csa):
    L = csa._lib
    rc = L.csa_compress(None, None, 0, 8, 0, 512, 10000.0, 0, _kv(csa), None)
    assert rc == csa.CSA_EUNSUPPORTED and b"m=0" in L.csa_last_error()
    rc = L.csa_compress(None, None, 0, 8, 4, 256, 10000.0, 0, _kv(csa), None)
    assert rc == csa.CSA_EUNSUPPORTED
    rc = L.csa_compress(None, None, 2, 8, 4, 512, 10000.0, 0, _kv(csa), None)
    assert rc == csa.CSA_EINVAL and b"complete blocks" in L.csa_last_error()
    rc = L.csa_compress(None, None, 0, 0, 4, 512, 10000.0, 0, _kv(csa), None)
    assert rc == csa.CSA_OK  # empty call is a no-op
    rc = L.csa_compress(ctypes.c_void_p(16), ctypes.c_void_p(16), 0, 8, 4, 512, 10000.0, 0, _kv(csa), None)
    assert rc == csa.CSA_EINVAL and b"null array" in L.csa_last_error()


def test_compress_variants_validation(csa):
    L = csa._lib
    p = ctypes.c_void_p(256)
    rc = L.csa_compress_channel(None, None, 0, 8, 0, 512, 10000.0, 0, _kv(csa), None)
    assert rc == csa.CSA_EUNSUPPORTED and b"m=0" in L.csa_last_error()
    rc = L.csa_compress_channel(p, p, 2, 8, 4, 512, 10000.0, 0, _kv(csa), None)
    assert rc == csa.CSA_EINVAL and b"complete blocks" in L.csa_last_error()
    rc = L.csa_compress_channel(None, None, 0, 0, 4, 512, 10000.0, 0, _kv(csa), None)
    assert rc == csa.CSA_OK  # empty call is a no-op
    keys = csa._IdxKeys(256, 256, 16)
    rc = L.csa_compress_index_keys(p, p, 0, 8, 4, 96, 0, keys, None)
    assert rc == csa.CSA_EUNSUPPORTED and b"d_i=96" in L.csa_last_error()
    rc = L.csa_compress_index_keys(p, p, 0, 6, 4, 128, 0, keys, None)
    assert rc == csa.CSA_EINVAL and b"complete blocks" in L.csa_last_error()
    rc = L.csa_compress_index_keys(p, p, 0, 128, 4, 128, 0, keys, None)
    assert rc == csa.CSA_EINVAL and b"out.cap" in L.csa_last_error()
    rc = L.csa_compress_index_keys(None, None, 0, 8, 4, 128, 0, csa._IdxKeys(None, None, 16), None)
    assert rc == csa.CSA_EINVAL and b"null" in L.csa_last_error()


def test_paged_cache_validation(csa):
    L = csa._lib
    p = ctypes.c_void_p(256)
    bad = csa._Kv(256, 256, 256, 96, 256, 24)  # page not a power of two
    rc = L.csa_compress(p, p, 0, 8, 4, 512, 10000.0, 0, bad, None)
    assert rc == csa.CSA_EINVAL and b"power of two" in L.csa_last_error()
    bad = csa._Kv(256, 256, 256, 96, 256, 64)  # page does not divide cap
    rc = L.csa_compress(p, p, 0, 8, 4, 512, 10000.0, 0, bad, None)
    assert rc == csa.CSA_EINVAL and b"divide" in L.csa_last_error()


def test_index_topk_validation(csa):
    L = csa._lib
    keys = csa._IdxKeys(None, None, 16)
    rc = L.csa_index_scores(None, None, None, None, None, 4, 16, 128, keys, 4, 16, None, None, 0, None)
    assert rc == csa.CSA_EUNSUPPORTED
    rc = L.csa_index_scores(None, None, None, None, None, 4, 8, 96, keys, 4, 16, None, None, 0, None)
    assert rc == csa.CSA_EUNSUPPORTED
    p = ctypes.c_void_p(256)
    rc = L.csa_index_scores(p, p, p, p, p, 4, 8, 128, csa._IdxKeys(256, 256, 8), 4, 16, p, None, 0, None)
    assert rc == csa.CSA_EINVAL and b"keys.cap" in L.csa_last_error()
    rc = L.csa_index_scores_grouped(p, p, p, p, p, 4, 8, 128, csa._IdxKeys(256, 256, 16), 4, 16, 3, p, None, 0, None)
    assert rc == csa.CSA_EUNSUPPORTED and b"group=3" in L.csa_last_error()
    rc = L.csa_index_scores_grouped(p, p, p, p, p, 6, 8, 128, csa._IdxKeys(256, 256, 16), 4, 16, 4, p, None, 0, None)
    assert rc == csa.CSA_EINVAL and b"multiple of group" in L.csa_last_error()
    rc = L.csa_index_scores_grouped(p, p, p, p, p, 4, 8, 128, csa._IdxKeys(256, 256, 8), 4, 16, 2, p, None, 0, None)
    assert rc == csa.CSA_EINVAL and b"keys.cap" in L.csa_last_error()
    rc = L.csa_index_scores_grouped(None, None, None, None, None, 0, 8, 128, keys, 4, 16, 2, None, None, 0, None)
    assert rc == csa.CSA_OK  # empty call is a no-op
    rc = L.csa_topk(None, 4, 100, None, 4, 0, None, None, 0, 0, None)
    assert rc == csa.CSA_EUNSUPPORTED
    rc = L.csa_topk(None, 4, 100, None, 4, 4096, None, None, 0, 0, None)
    assert rc == csa.CSA_EUNSUPPORTED
    rc = L.csa_topk(None, 0, 100, None, 4, 64, None, None, 0, 0, None)
    assert rc == csa.CSA_OK
    rc = L.csa_topk(p, 4, 100, p, 4, 64, p, None, 0, 8, None)
    assert rc == csa.CSA_EINVAL and b"flags" in L.csa_last_error()


def test_mqa_validation(csa):
    L = csa._lib
    p = ctypes.c_void_p(256)
    kv = csa._Kv(256, 256, 256, 256)
    args = dict(T=2, H=64, d=512, k=64, m=4, window=128)

    def sparse(**o):
        a = dict(args, **o)
        return L.csa_sparse_mqa(p, p, p, a["T"], a["H"], a["d"], p, a["k"], a["m"], kv, a.get("win", kv),
                                a["window"], 0.04, 10000.0, p, p, None, 0, None)

    assert sparse(H=48) == csa.CSA_EUNSUPPORTED
    assert sparse(d=256) == csa.CSA_EUNSUPPORTED
    assert sparse(k=4096) == csa.CSA_EUNSUPPORTED
    assert sparse(window=2000) == csa.CSA_EUNSUPPORTED
    assert sparse(win=csa._Kv(256, 256, 256, 16)) == csa.CSA_EINVAL  # ring smaller than the window
    assert sparse(T=0) == csa.CSA_OK
    rc = L.hca_dense_mqa(p, p, p, 2, 64, 512, 128, 0, kv, kv, 128, 0.04, 10000.0, p, p, None, 0, None)
    assert rc == csa.CSA_EINVAL and b"max_vis" in L.csa_last_error()
    rc = L.hca_dense_mqa(p, p, p, 2, 64, 512, 128, 8192, kv, kv, 128, 0.04, 10000.0, p, p, None, 0, None)
    assert rc == csa.CSA_EWORKSPACE


def test_mqa_bwd_validation(csa):
    L = csa._lib
    p = ctypes.c_void_p(256)
    kv = csa._Kv(256, 256, 256, 256)
    args = dict(T=2, H=64, d=512, k=64, m=4, window=128)

    def bwd(**o):
        a = dict(args, **o)
        return L.csa_mqa_bwd(p, p, p, a["T"], a["H"], a["d"], a.get("idx", p), a["k"], a["m"], kv, kv, a["window"],
                             0.04, 10000.0, a.get("out", p), p, p, p, p, a.get("comp_rows", 100), a.get("dwin", p),
                             a.get("win_rows", 100), a.get("ws", p), a.get("ws_bytes", 1 << 30), None)

    assert bwd(d=128) == csa.CSA_EUNSUPPORTED and b"d=128" in L.csa_last_error()
    assert bwd(comp_rows=0) == csa.CSA_EINVAL and b"comp_rows" in L.csa_last_error()
    assert bwd(ws_bytes=100) == csa.CSA_EWORKSPACE
    assert bwd(ws=ctypes.c_void_p(260)) == csa.CSA_EINVAL and b"8-byte" in L.csa_last_error()
    assert csa.csa_mqa_bwd_workspace(100, 100, 512) == 200 * 512 * 8
    assert bwd(H=48) == csa.CSA_EUNSUPPORTED
    assert bwd(k=4096) == csa.CSA_EUNSUPPORTED
    assert bwd(out=None) == csa.CSA_EINVAL
    assert bwd(dwin=None) == csa.CSA_EINVAL  # window > 0 needs the window gradient
    assert bwd(out=ctypes.c_void_p(264)) == csa.CSA_EINVAL and b"aligned" in L.csa_last_error()
    assert bwd(T=0) == csa.CSA_OK


def test_workspace_sizes(csa):
    assert csa.csa_topk_workspace(4, 262144, 1024) >= 0
    # decode shapes split the key list; big batches do not
    assert csa.csa_mqa_workspace(4, 64, 512, 1152) > 0
    assert csa.csa_mqa_workspace(8192, 64, 512, 1152) == 0


def test_index_topk_and_index_bwd_validation(csa):
    L = csa._lib
    p = ctypes.c_void_p(256)
    keys = csa._IdxKeys(256, 256, 4096)
    # csa_index_topk: k range, workspace
    rc = L.csa_index_topk(p, p, p, p, p, 4, 8, 128, keys, 4, 4096, 4096, p, p, 1 << 30, None)
    assert rc == csa.CSA_EUNSUPPORTED and b"k=4096" in L.csa_last_error()
    rc = L.csa_index_topk(p, p, p, p, p, 4, 8, 128, keys, 4, 4096, 1024, p, p, 16, None)
    assert rc == csa.CSA_EWORKSPACE
    rc = L.csa_index_topk(p, p, p, p, p, 4, 8, 96, keys, 4, 4096, 1024, p, p, 1 << 30, None)
    assert rc == csa.CSA_EUNSUPPORTED
    assert csa.csa_index_topk_workspace(4, 262144, 1024, 8) > 0
    assert csa.csa_index_topk_workspace(4, 262144, 4096, 8) == 0
    # csa_index_bwd: shapes, workspace
    rc = L.csa_index_bwd(p, p, p, p, p, 4, 8, 128, keys, 4, p, p, 0, p, p, p, 100, p, 1 << 30, None)
    assert rc == csa.CSA_EINVAL and b"n_sel" in L.csa_last_error()
    rc = L.csa_index_bwd(p, p, p, p, p, 4, 8, 128, keys, 4, p, p, 16, p, p, p, 100, p, 64, None)
    assert rc == csa.CSA_EWORKSPACE
    rc = L.csa_index_bwd(p, p, p, p, p, 4, 3, 128, keys, 4, p, p, 16, p, p, p, 100, p, 1 << 30, None)
    assert rc == csa.CSA_EUNSUPPORTED
    assert csa.csa_index_bwd_workspace(100, 128) == 100 * 128 * 8


def test_mfma_probe_validation(csa):
    lib = csa._lib
    assert lib.csa_mfma_probe_flops(0, 2, 8) == 16 * 16 * 32 * 2 * 4 * 8 * 2 * 4
    assert lib.csa_mfma_probe_flops(1, 1, 4) == 32 * 32 * 64 * 2 * 4 * 4 * 4
    assert lib.csa_mfma_probe_flops(0, 1, 6) == -1
    assert lib.csa_mfma_probe_flops(2, 1, 1) == -1
    assert lib.csa_mfma_probe_flops(0, 0, 1) == -1
    assert lib.csa_mfma_probe(2, 1, 4, None, 256, None) == -2
    assert lib.csa_mfma_probe(0, 1, 4, None, 256, None) == -1
    assert b"sink" in lib.csa_last_error()


def test_pages_copy_validation(csa):
    """csa_pages_store / csa_pages_load refuse bad arguments before any copy is enqueued: a
    negative page number anywhere in the list, a host buffer too small, a page size that is
    not a power of two, index keys on another page size."""
    L = csa._lib
    p = ctypes.c_void_p(256)
    kv = csa._Kv(256, 256, 256, 1024, None, 64)
    keys = csa._IdxKeys(256, 256, 1024, None, 64)
    per = L.csa_pages_bytes(64, 512, 128)
    assert per == 64 * (448 + 128 + 4 + 64 + 4)
    pages = (ctypes.c_int32 * 3)(0, 5, -1)
    host = ctypes.create_string_buffer(3 * per)
    rc = L.csa_pages_store(kv, keys, 512, 128, pages, 3, host, 3 * per, None)
    assert rc == csa.CSA_EINVAL and b"negative page number at 2" in L.csa_last_error()
    rc = L.csa_pages_load(kv, keys, 512, 128, pages, 3, host, 3 * per, None)
    assert rc == csa.CSA_EINVAL and b"negative page" in L.csa_last_error()
    ok_pages = (ctypes.c_int32 * 3)(0, 5, 1)
    rc = L.csa_pages_store(kv, keys, 512, 128, ok_pages, 3, host, 3 * per - 1, None)
    assert rc == csa.CSA_EWORKSPACE
    rc = L.csa_pages_store(csa._Kv(256, 256, 256, 1024, None, 48), keys, 512, 128, ok_pages, 3, host, 3 * per, None)
    assert rc == csa.CSA_EINVAL and b"power of two" in L.csa_last_error()
    rc = L.csa_pages_store(kv, csa._IdxKeys(256, 256, 1024, None, 32), 512, 128, ok_pages, 3, host, 3 * per, None)
    assert rc == csa.CSA_EINVAL and b"keys.page" in L.csa_last_error()
    assert L.csa_pages_store(kv, keys, 512, 128, ok_pages, 0, host, 0, None) == 0
