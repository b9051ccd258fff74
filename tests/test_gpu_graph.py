"""The decode step (indexer with row summary, top-k, sparse attention) captured
as HIP graphs, as bench.py times it: every replay, with eager library work
between the replays, equals the eager step bit for bit, and the eager step
equals the oracle."""
import sys

import numpy as np
import pytest

from gen import configs

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


def test_decode_step_graph_replays(lib, orc):
    import torch

    from bench import DecodeSet

    _say("decode step as a 3-step HIP graph, 2 replica sets, L = 524,288")
    wl = configs.named("csa_decode_1m", L=1 << 19)
    ds = DecodeSet(wl, replicas=2)
    want = ds.capture(3)
    scores = ds.scores.clone()
    ref_s = orc.index_scores(wl["iq"][0], wl["iq"][1], wl["w"], wl["seq"], wl["pos"], wl["keys"][0], wl["keys"][1],
                             wl["N"], wl["m"], wl["n_cols"]).astype(np.float32)
    assert np.array_equal(scores.cpu().numpy().view(np.uint32), ref_s.view(np.uint32))
    assert np.array_equal(want[0].cpu().numpy(), orc.topk(ref_s, wl["pos"], wl["m"], wl["k"]))
    other = torch.rand(3, 5000, device="cuda")
    opos = torch.full((3,), 4 * 5000 - 1, dtype=torch.int64, device="cuda")
    for i in range(6):
        ds.idx.fill_(-5)
        ds.out.fill_(1.0)
        ds.scores.zero_()
        lib.csa_topk(other, opos, 4, 100)  # eager library work between replays
        ds.graph.replay()
        ds.check(want, f"replay {i}")
        assert torch.equal(ds.scores, scores), f"replay {i}: scores"
        ds.step(i)  # and eager steps on the same buffers
        ds.check(want, f"eager step after replay {i}")
