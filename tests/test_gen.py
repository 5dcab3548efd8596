"""The seeded generator: determinism, prefix stability, encoding rule."""
import numpy as np

import pins


def test_deterministic_and_prefix_stable(genlib):
    g = genlib
    a = g.idx_rows(g.seed(1), 0, 300)
    b = g.idx_rows(g.seed(1), 0, 120)
    assert np.array_equal(a[:120], b)
    assert np.array_equal(g.idx_rows(g.seed(1), 0, 50, row0=100), a[100:150])
    kv = g.kv_rows(g.seed(1), 0, 64)
    assert np.array_equal(g.kv_rows(g.seed(1), 0, 16, row0=48), kv[48:])
    assert g.digest(a) == g.digest(g.idx_rows(g.seed(1), 0, 300))
    assert g.digest(g.idx_rows(g.seed(1), 1, 300)) != g.digest(a)  # sessions differ
    assert g.digest(g.idx_rows(g.seed(2), 0, 300)) != g.digest(a)  # workloads differ


def test_distributions(genlib):
    g = genlib
    sd = g.seed(0)
    z = np.array([g.lib().csa_gen_normal(sd, 3, i) for i in range(20000)])
    assert abs(z.mean()) < 0.03 and abs(z.std() - 1) < 0.03
    u = np.array([g.lib().csa_gen_uniform(sd, 4, i) for i in range(20000)])
    assert u.min() >= 0 and u.max() < 1 and abs(u.mean() - 0.5) < 0.01
    q_idx, w, q_attn = g.queries(sd, 0, 8, 64)
    assert q_idx.shape == (8, 128) and w.shape == (8,) and q_attn.shape == (64, 512)
    assert np.all((w >= 0) & (w < 1))


def _nearest_grid_ok(x, decoded, grid):
    # decoded must be a nearest grid point of x (ties either way)
    d_best = np.min(np.abs(np.abs(x)[:, None] - grid[None, :]), axis=1)
    return np.all(np.abs(np.abs(decoded) - np.abs(x)) <= d_best + 1e-12)


def test_indexer_encoding_rule(genlib):
    g = genlib
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)
    rng = np.random.default_rng(0)
    for trial in range(200):
        v = (rng.standard_normal(128) * 2.0 ** rng.integers(-10, 10)).astype(np.float32)
        if trial % 7 == 0:
            v[:32] = 0  # an all-zero block
        row = g.pack_idx_row(v)
        dec = pins.ref_decode_idx(row)[0].astype(np.float64)
        for b in range(4):
            blk = v[32 * b:32 * b + 32].astype(np.float64)
            amax = np.abs(blk).max()
            exp_byte = 127 if amax == 0 else int(np.clip(np.floor(np.log2(amax)) - 2 + 127, 0, 254))
            assert row[64 + b] == exp_byte
            scale = 2.0 ** (exp_byte - 127)
            xs = np.minimum(np.abs(blk) / scale, 6.0)
            assert _nearest_grid_ok(xs, dec[32 * b:32 * b + 32] / scale, grid)
            assert np.all((dec[32 * b:32 * b + 32] == 0) | (np.sign(dec[32 * b:32 * b + 32]) == np.sign(blk)))


def test_kv_encoding_rule(genlib):
    g = genlib
    e4m3 = np.unique(np.abs(pins.lib_e4m3(np.arange(256))))
    e4m3 = e4m3[~np.isnan(e4m3)]
    rng = np.random.default_rng(1)
    for trial in range(50):
        v = (rng.standard_normal(512) * 2.0 ** rng.integers(-20, 20)).astype(np.float32)
        row = g.pack_kv_row(v)
        dec = pins.ref_decode_kv(row)[0].astype(np.float64)
        for b in range(7):
            blk = v[64 * b:64 * b + 64].astype(np.float64)
            amax = np.abs(blk).max()
            exp_byte = int(np.clip(np.floor(np.log2(amax)) - 8 + 127, 0, 254))
            assert row[576 + b] == exp_byte
            scale = 2.0 ** (exp_byte - 127)
            xs = np.minimum(np.abs(blk) / scale, 448.0)
            assert _nearest_grid_ok(xs, dec[64 * b:64 * b + 64] / scale, e4m3)
        with np.errstate(over="ignore"):
            rope = v[448:].astype(np.float16).astype(np.float32)
        assert np.array_equal(dec[448:].astype(np.float32), rope)  # FP16 round-to-nearest-even
