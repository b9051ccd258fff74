"""Input generator: determinism, row slicing, encoding sanity (inputs only)."""
import numpy as np

from gen import configs


def test_counter_rng_is_deterministic_and_sliceable(gen):
    a = gen.normal_bf16(7, 3, (1000,))
    b = gen.normal_bf16(7, 3, (1000,))
    assert np.array_equal(a, b)
    assert not np.array_equal(a, gen.normal_bf16(7, 4, (1000,)))
    d1, s1, _ = gen.mxfp4(7, 5, 64, 128)
    d2, s2, _ = gen.mxfp4(7, 5, 16, 128, row0=40)
    assert np.array_equal(d1[40:56], d2) and np.array_equal(s1[40:56], s2)
    e1 = gen.entries(7, 6, 32, 448)
    e2 = gen.entries(7, 6, 8, 448, row0=20)
    assert all(np.array_equal(x[20:28], y) for x, y in zip(e1, e2))


def test_normal_moments(gen):
    x = gen.normal_f32(9, 1, (200000,)).astype(np.float64)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01


def test_mxfp4_encoding_tracks_values(gen, orc):
    d, s, _ = gen.mxfp4(8, 1, 256, 128)
    ref = np.array([[gen._load().gen_normal(8, 1, r * 128 + c) for c in range(128)] for r in range(256)])
    lo = d & 15
    hi = d >> 4
    nib = np.stack([lo, hi], axis=-1).reshape(256, 128)
    tab = np.array([orc.e2m1_to_f64(c) for c in range(16)])
    val = tab[nib] * np.repeat(2.0 ** (s.astype(np.float64) - 127), 32, axis=1)
    # E2M1 keeps ~1 significant bit: error bounded by half a grid step at the block scale
    blk = np.repeat(2.0 ** (s.astype(np.float64) - 127), 32, axis=1)
    assert np.all(np.abs(val - ref) <= 1.0 * blk + 2.0 * blk * (np.abs(ref) > 6 * blk))
    amax = np.abs(ref).reshape(256, 4, 32).max(axis=2)
    assert np.array_equal(s.astype(int) - 127, np.floor(np.log2(amax)).astype(int) - 2)


def test_planted_fraction(gen):
    _, _, planted = gen.mxfp4(104, 22, 40000, 128, plant_frac=0.05)
    assert abs(planted.mean() - 0.05) < 0.005


def test_workload_shapes_small():
    wl = configs.named("prefill_small")
    assert wl["kv"].shape == (2048, 128) and wl["q"].shape == (2048, 16, 128)
    assert wl["iq"][0].shape == (2048, 4, 32) and wl["keys"][0].shape == (512, 32)
    wl = configs.csa_decode(B=2, L=4096, plant_frac=0.05)
    assert wl["comp"][0].shape == (2048, 448) and wl["win"][1].shape == (256, 64)
