"""The synthetic workload generator lands on its stated statistics and is reproducible."""
import os

import numpy as np
import torch

import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(10000).astype(np.float32) * 100,
                        np.array([0.0, -0.0, 1.0, -1.5, 3.0e38, 1e-40, np.inf, -np.inf], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(synth.f32_to_bf16_bits(x), ref)
    back = synth.bf16_bits_to_f32(ref)
    np.testing.assert_array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


def golden_values(name):
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", name)
    with open(path) as f:
        return {k: float(v) for k, v in (line.split() for line in f if line.strip() and not line.startswith("#"))}


def test_loop_and_channel_correlations():
    """The generator's loop-step and cross-channel correlations are the ones the pages
    report for Ouro-1.4B (tests/golden/loop_statistics.txt)."""
    pages = golden_values("loop_statistics.txt")
    rng = np.random.default_rng(1)
    H, d, N = 2, 64, 20000
    sc = np.ones((H, d))
    for T in (4, 8):
        X = synth.gen_kv(rng, T, N, H, d, sc).astype(np.float64)
        rho = synth.loop_rhos(T)
        assert rho[0] == pages["first_pair_step_correlation"]
        assert abs(rho[-1] - pages["last_pair_step_correlation"]) < 1e-12
        for t in range(1, T):
            r = np.mean([np.corrcoef(X[t - 1, :, 0, j], X[t, :, 0, j])[0, 1] for j in range(8)])
            assert abs(r - rho[t - 1]) < 0.02
        cc = np.corrcoef(X[T - 1, :, 1, :8].T)
        off = cc[~np.eye(8, dtype=bool)].mean()
        assert abs(off - pages["cross_channel_correlation"]) < 0.02


def test_scales_and_outliers():
    rng = np.random.default_rng(2)
    s = synth.channel_scales(rng, 16, 128)
    for h in range(16):
        big = np.sort(s[h])[-2:]
        assert big.min() > 2.0 and np.median(s[h]) < 1.5
    assert abs(np.log(s[s < 4]).std() - 0.5) < 0.08


def test_reproducible_and_page_tables():
    a = synth.gen_queries(np.random.default_rng(synth.seed_for(2, synth.STREAM_Q)), 4, 2, 3, 8)
    b = synth.gen_queries(np.random.default_rng(synth.seed_for(2, synth.STREAM_Q)), 4, 2, 3, 8)
    np.testing.assert_array_equal(a, b)
    tab, pool = synth.shuffled_page_table(np.random.default_rng(3), [5, 0, 7], 9)
    used = tab[tab >= 0]
    assert pool == 12 and sorted(used.tolist()) == list(range(12))
    assert np.all(tab[1] == -1)


def test_pack_bf16_pages_layout():
    rng = np.random.default_rng(4)
    T, H, d = 2, 3, 8
    ks = [rng.integers(0, 1 << 16, size=(T, L, H, d), dtype=np.uint16) for L in (21, 40)]
    vs = [rng.integers(0, 1 << 16, size=(T, L, H, d), dtype=np.uint16) for L in (21, 40)]
    q_end = np.array([8, 16])
    pool, lay = synth.pack_bf16_pages(ks, vs, q_end, T, H, d, rng=np.random.default_rng(5))
    for b, L in enumerate((21, 40)):
        row = lay.bf16_table[b]
        np.testing.assert_array_equal(pool[row[0], :, :, 0, :8], ks[b][:, 0:8].transpose(0, 2, 1, 3))
        for p in range(int(q_end[b]), L):
            pg = row[1 + p // 8 - int(q_end[b]) // 8]
            np.testing.assert_array_equal(pool[pg, :, :, 1, p % 8], vs[b][:, p])


def test_kmeans_fixture_is_deterministic_and_fits():
    rng = np.random.default_rng(6)
    T, Tc, G, H, d = 4, 2, 16, 1, 16
    sc = synth.channel_scales(rng, H, d)
    cb1 = synth.kmeans_codebooks(7, T, Tc, G, H, d, sc, sc, n_samples=1024)
    cb2 = synth.kmeans_codebooks(7, T, Tc, G, H, d, sc, sc, n_samples=1024)
    np.testing.assert_array_equal(cb1, cb2)
    assert cb1.shape == (2, 2, 1, 2, 2, 256, 8)
    # the codewords live on the data's scale (not degenerate)
    v = synth.bf16_bits_to_f32(cb1).astype(np.float64)
    assert np.isfinite(v).all() and v.std() > 0.3
