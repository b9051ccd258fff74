"""The entry point that allocates nothing (csa_topk_noalloc), through the C ABI,
against csa_topk with a caller workspace: identical indices on two calls in a
row, the second with a smaller input (the shared scratch array keeps the first
call's contents), on the row-summary path that uses the scratch and on a path
that needs none; a shape beyond the array's size is refused."""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def lib():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import compressed_sparse_long_compress_amd as csa

    return csa


def _scores(rng, T, n):
    s = np.abs(rng.standard_normal((T, n))).astype(np.float32) * 10
    s[:, ::97] = 3.0  # repeated values: ties resolved toward the lower column
    return s


@pytest.mark.parametrize("first,second", [
    ((4, 262144, 1024), (2, 100000, 512)),    # both select from the row summary (scratch in use)
    ((8, 100000, 2048), (3, 70000, 1)),
    ((130, 20000, 1024), (4, 70000, 1024)),   # a shape that needs no scratch, then one that does
])
def test_noalloc_matches_workspace_call(lib, first, second):
    import torch

    from gen import device as dev

    rng = np.random.default_rng(sum(first) + sum(second))
    for (T, n, k) in (first, second):
        _say(f"topk_noalloc T={T} n_cols={n} k={k}")
        sc = dev.t(_scores(rng, T, n))
        pos = np.full(T, 4 * n - 1, np.int64)
        pos[-1] = 4 * (n // 2) + 1  # a shorter row
        tpos = dev.t(pos)
        want = lib.csa_topk(sc, tpos, 4, k)
        got = lib.csa_topk_noalloc(sc, tpos, 4, k)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"T={T} n_cols={n} k={k}: indices differ"


def test_noalloc_refuses_shapes_beyond_its_scratch(lib):
    import torch

    from gen import device as dev

    _say("topk_noalloc refuses an oversized shape")
    T, n, k = 100, 1 << 21, 1024  # row summaries alone would need 26 MB
    assert lib.csa_topk_workspace(T, n, k) > 12 << 20
    sc = torch.empty(T, n, dtype=torch.float32, device="cuda")
    pos = dev.t(np.full(T, 4 * n - 1, np.int64))
    with pytest.raises(lib.CsaError) as e:
        lib.csa_topk_noalloc(sc, pos, 4, k)
    assert e.value.code == lib.CSA_EUNSUPPORTED and "scratch" in str(e.value)
