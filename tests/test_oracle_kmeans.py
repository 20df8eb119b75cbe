"""Pins of the codebook-builder oracle (k-means++ seeding, Lloyd iterations, bf16 rounding)
against what the mathematics and independent routines fix."""
import numpy as np
import pytest

from oracle import lvq_oracle as orc


def test_round_bf16_nearest_even():
    # bf16 keeps 8 significant bits: 1 + k/128 is exact, halfway cases go to the even neighbour
    one = 1.0
    ulp = 2.0 ** -7
    assert orc.round_bf16(np.array([one + ulp]))[0] == one + ulp
    assert orc.round_bf16(np.array([one + ulp / 2]))[0] == one              # tie -> even (1.0)
    assert orc.round_bf16(np.array([one + 3 * ulp / 2]))[0] == one + 2 * ulp  # tie -> even
    assert orc.round_bf16(np.array([one + ulp / 2 + 2.0 ** -20]))[0] == one + ulp
    assert orc.round_bf16(np.array([-(one + 3 * ulp / 2)]))[0] == -(one + 2 * ulp)
    # float64 -> float32 first: a value just above a bf16 tie that float32 rounds onto the tie
    v = one + ulp / 2 + 2.0 ** -40
    assert np.float32(v) == np.float32(one + ulp / 2)
    assert orc.round_bf16(np.array([v]))[0] == one
    bits = orc.bf16_bits_of(np.array([1.0, -2.0, 0.5]))
    assert list(bits) == [0x3F80, 0xC000, 0x3F00]


def test_kmeanspp_hand_case():
    # D^2 sampling worked by hand: picks sample 2 (floor(0.6*4)), then with D^2 = [9,4,0,49],
    # cumulative [9,13,13,62] and target 0.5*62 = 31 -> sample 3, then D^2 = [9,4,0,0],
    # cumulative [9,13,13,13], target 0.7*13 = 9.1 -> sample 1.
    X = np.array([[0.], [1.], [3.], [10.]])
    assert list(orc.kmeanspp_seed(X, np.array([0.6, 0.5, 0.7]), K=3)) == [2, 3, 1]
    # u = 0 picks the first sample with positive D^2, never a chosen one
    assert list(orc.kmeanspp_seed(X, np.array([0.0, 0.0, 0.0]), K=3)) == [0, 1, 2]
    # all samples equal: every D^2 is 0 and the fallback floor(u*S) applies
    Z = np.zeros((5, 2))
    assert list(orc.kmeanspp_seed(Z, np.array([0.1, 0.5, 0.99]), K=3)) == [0, 2, 4]


def test_kmeanspp_picks_every_distinct_sample_once():
    # S = K distinct samples: a chosen sample has D^2 = 0 and cannot be picked again, so the
    # seeding is a permutation of the samples starting at floor(u_0 * S)
    rng = np.random.default_rng(3)
    X = rng.standard_normal((256, 8))
    draws = rng.random(256)
    picks = orc.kmeanspp_seed(X, draws)
    assert sorted(picks) == list(range(256))
    assert picks[0] == int(draws[0] * 256)


def test_distinct_samples_are_a_fixed_point():
    # with S = K the Lloyd iterations keep each center on its own sample: the book is the
    # sample set (rounded to bf16: the samples are bf16 already) in seeding order
    rng = np.random.default_rng(4)
    X = orc.round_bf16(rng.standard_normal((256, 16)))
    draws = rng.random(256)
    picks = orc.kmeanspp_seed(X, draws)
    C = orc.lloyd(X, X[picks], 5)
    np.testing.assert_array_equal(C, X[picks])


def test_lloyd_matches_scikit_learn():
    # plain float64 Lloyd from the same initial centers = scikit-learn's Lloyd iterations
    from sklearn.cluster import KMeans
    rng = np.random.default_rng(5)
    K, G, per = 16, 4, 20
    means = rng.standard_normal((K, G)) * 10
    X = np.concatenate([m + rng.standard_normal((per, G)) for m in means])
    init = X[np.arange(K) * per + 3]          # one point of each blob: no cluster empties
    ours = orc.lloyd(X, init, 6, bf16_assign=False)
    km = KMeans(n_clusters=K, init=init, n_init=1, max_iter=6, tol=0.0, algorithm="lloyd").fit(X)
    np.testing.assert_allclose(ours, km.cluster_centers_, rtol=0, atol=1e-12)


def test_lloyd_update_is_member_mean_and_assignment_is_nearest():
    # the assignment sees the centers rounded to bf16: 1 + 2^-9 rounds to 1, so the midpoint
    # moves from 1.5 + 2^-10 to 1.5 and the sample 1.5 + 2^-11 goes to the second center
    x = np.array([[1.5 + 2.0 ** -11]])
    C1 = orc.lloyd(x, np.array([[1.0 + 2.0 ** -9], [2.0]]), 1)
    np.testing.assert_array_equal(C1, [[1.0 + 2.0 ** -9], [1.5 + 2.0 ** -11]])
    rng = np.random.default_rng(6)
    X = orc.round_bf16(rng.standard_normal((600, 8)))
    C0 = X[rng.choice(600, 32, replace=False)]
    C1 = orc.lloyd(X, C0, 1)
    A = orc.round_bf16(C0)
    dist = np.linalg.norm(X[:, None, :] - A[None, :, :], axis=2)
    assign = np.argmin(dist, axis=1)
    for k in range(32):
        m = assign == k
        if m.any():
            np.testing.assert_allclose(C1[k], X[m].mean(axis=0), rtol=0, atol=1e-14)
        else:
            np.testing.assert_array_equal(C1[k], C0[k])


def test_empty_cluster_keeps_its_center():
    X = np.array([[0.0, 0.0], [0.0, 1.0], [1.0, 0.0]])
    C0 = np.array([[0.0, 0.0], [100.0, 100.0]])     # the far center attracts no sample
    C1 = orc.lloyd(X, C0, 1)
    np.testing.assert_allclose(C1[0], [1 / 3, 1 / 3])
    np.testing.assert_array_equal(C1[1], [100.0, 100.0])


def test_build_codebooks_layout_and_shape():
    # two blocks (Tc = 2 of T = 4), G = 16 -> c = 8, d = 16 -> 2 groups, H = 1; S = K distinct
    # joint vectors: each book is its samples' joint vectors in seeding order, split per step
    rng = np.random.default_rng(7)
    T, S, H, d, Tc, G = 4, 256, 1, 16, 2, 16
    x = orc.round_bf16(rng.standard_normal((T, S, H, d)))
    bits = orc.bf16_bits_of(x)
    draws = rng.random((2, H, 2, 256))
    books = orc.build_codebooks(bits, draws, Tc, G, n_iter=2)
    assert books.shape == (2, H, 2, Tc, 256, 8)
    J = orc.joint_vectors(x, Tc, G)
    for beta in range(2):
        for g in range(2):
            picks = orc.kmeanspp_seed(J[beta, :, 0, g], draws[beta, 0, g])
            want = orc.bf16_bits_of(J[beta, picks, 0, g])
            for tau in range(Tc):
                np.testing.assert_array_equal(books[beta, 0, g, tau], want[:, tau * 8:(tau + 1) * 8])


@pytest.mark.parametrize("mutant", ["ge_not_gt", "highest_tie", "empty_to_zero", "ceil_first",
                                    "d2_last_center_only", "assign_unrounded"])
def test_kmeans_mutants_are_caught(mutant, monkeypatch):
    """Plausible mistakes planted in the oracle (on the CPU) fail one of the pins above."""
    def seed_mut(X, draws, K=orc.NCODES):
        S = X.shape[0]
        picks = np.empty(K, dtype=np.int64)
        first = int(np.ceil(draws[0] * S)) if mutant == "ceil_first" else int(draws[0] * S)
        picks[0] = min(first, S - 1)
        D2 = orc.sq_dist_sequential(X, X[picks[0]])
        for k in range(1, K):
            cum = np.cumsum(D2)
            total = cum[-1]
            if total > 0:
                target = draws[k] * total
                above = np.flatnonzero(cum >= target) if mutant == "ge_not_gt" else np.flatnonzero(cum > target)
                i = int(above[0]) if len(above) else int(np.flatnonzero(D2 > 0)[-1])
            else:
                i = min(int(draws[k] * S), S - 1)
            picks[k] = i
            D2i = orc.sq_dist_sequential(X, X[i])
            D2 = D2i if mutant == "d2_last_center_only" else np.minimum(D2, D2i)
        return picks

    def lloyd_mut(X, centers, n_iter, bf16_assign=True):
        C = np.array(centers, dtype=np.float64)
        K, G = C.shape
        for _ in range(n_iter):
            A = orc.round_bf16(C) if bf16_assign and mutant != "assign_unrounded" else C
            D = ((X[:, None, :] - A[None]) ** 2).sum(-1)
            assign = (K - 1 - np.argmin(D[:, ::-1], axis=1)) if mutant == "highest_tie" else np.argmin(D, axis=1)
            new = C.copy()
            for k in range(K):
                m = np.flatnonzero(assign == k)
                if len(m):
                    new[k] = X[m].mean(axis=0)
                elif mutant == "empty_to_zero":
                    new[k] = 0.0
            C = new
        return C

    monkeypatch.setattr(orc, "kmeanspp_seed", seed_mut)
    monkeypatch.setattr(orc, "lloyd", lloyd_mut)
    failed = 0
    checks = [test_kmeanspp_hand_case, test_empty_cluster_keeps_its_center,
              test_kmeanspp_picks_every_distinct_sample_once,
              test_lloyd_update_is_member_mean_and_assignment_is_nearest]
    if mutant == "highest_tie":
        # duplicate centers tie exactly: the lowest index must win
        def tie_check():
            X = np.array([[0.0], [5.0]])
            C = orc.lloyd(X, np.array([[0.0], [0.0], [5.0]]), 1)
            np.testing.assert_array_equal(C, [[0.0], [0.0], [5.0]])
            C = orc.lloyd(np.array([[1.0]]), np.array([[0.0], [0.0]]), 1)
            np.testing.assert_array_equal(C, [[1.0], [0.0]])
        checks = [tie_check]
    for chk in checks:
        try:
            chk()
        except AssertionError:
            failed += 1
    assert failed >= 1, f"mutant {mutant} not caught"


def test_lowest_index_tie_in_lloyd():
    # duplicate centers: the member goes to the lower index, the duplicate keeps its place
    C = orc.lloyd(np.array([[1.0]]), np.array([[0.0], [0.0]]), 1)
    np.testing.assert_array_equal(C, [[1.0], [0.0]])


# ---------------------------------------------------------------- weighted k-means
def test_weighted_lloyd_matches_scikit_learn():
    # weighted Lloyd from the same initial centers = scikit-learn's with sample_weight
    from sklearn.cluster import KMeans
    rng = np.random.default_rng(8)
    K, G, per = 12, 4, 25
    means = rng.standard_normal((K, G)) * 10
    X = np.concatenate([m + rng.standard_normal((per, G)) for m in means])
    w = rng.uniform(0.1, 3.0, len(X))
    init = X[np.arange(K) * per + 5]
    ours = orc.lloyd(X, init, 6, bf16_assign=False, w=w)
    km = KMeans(n_clusters=K, init=init, n_init=1, max_iter=6, tol=0.0, algorithm="lloyd").fit(X, sample_weight=w)
    np.testing.assert_allclose(ours, km.cluster_centers_, rtol=0, atol=1e-12)
    # the weights matter: the unweighted means differ
    plain = orc.lloyd(X, init, 6, bf16_assign=False)
    assert np.abs(plain - ours).max() > 1e-3


def _integer_cloud(seed, S, G, lo=-20, hi=20):
    rng = np.random.default_rng(seed)
    X = rng.integers(lo, hi, (S, G)).astype(np.float64)
    return X, rng


def test_integer_weights_equal_duplicated_samples():
    # weight m on a sample = m copies of it: with integer coordinates every distance, running
    # sum, member sum and weight sum is exact, so seeding picks the same points (mapped back to
    # the original samples) and Lloyd yields the same centers to the bit
    K = 16
    X, rng = _integer_cloud(9, 120, 6)
    w = rng.integers(0, 4, len(X)).astype(np.float64)
    w[:3] = [0, 2, 3]
    rep = np.repeat(np.arange(len(X)), w.astype(int))
    Xd = X[rep]
    draws = rng.random(K)
    pw = orc.kmeanspp_seed(X, draws, K=K, w=w)
    pd = orc.kmeanspp_seed(Xd, draws, K=K)
    np.testing.assert_array_equal(pw, rep[pd])
    assert np.all(w[pw] > 0)
    Cw = orc.lloyd(X, X[pw], 4, w=w)
    Cd = orc.lloyd(Xd, Xd[pd], 4)
    np.testing.assert_array_equal(Cw, Cd)


def test_zero_weight_outliers_change_nothing():
    # samples of weight 0 are never seeds and add nothing to a mean, wherever they sit
    T, S, H, d, Tc, G = 2, 300, 1, 16, 2, 16
    rng = np.random.default_rng(10)
    x = orc.round_bf16(rng.standard_normal((T, S, H, d)))
    draws = rng.random((1, H, 2, 256))
    base = orc.build_codebooks(orc.bf16_bits_of(x), draws, Tc, G, 3)
    ins = np.sort(rng.choice(S + 40, 40, replace=False))
    keep = np.setdiff1d(np.arange(S + 40), ins)
    y = np.zeros((T, S + 40, H, d))
    y[:, keep] = x
    y[:, ins] = orc.round_bf16(50.0 + 10 * rng.standard_normal((T, 40, H, d)))
    w = np.ones((1, S + 40, H, 2))
    w[:, ins] = 0.0
    out = orc.build_codebooks(orc.bf16_bits_of(y), draws, Tc, G, 3, weights=w)
    np.testing.assert_array_equal(out, base)
    # unit weights are the unweighted build
    np.testing.assert_array_equal(orc.build_codebooks(orc.bf16_bits_of(x), draws, Tc, G, 3,
                                                      weights=np.ones((1, S, H, 2))), base)


@pytest.mark.parametrize("mutant", ["seed_ignores_weight", "first_pick_uniform", "mean_over_count"])
def test_weighted_mutants_are_caught(mutant, monkeypatch):
    """Plausible mistakes in the weighted builder, planted in the oracle on the CPU, fail a pin."""
    real_pick, real_lloyd = orc._running_sum_pick, orc.lloyd

    def seed_mut(X, draws, K=orc.NCODES, w=None):
        S = X.shape[0]
        wv = np.ones(S) if w is None else np.asarray(w, dtype=np.float64)
        picks = np.empty(K, dtype=np.int64)
        picks[0] = real_pick(np.ones(S) if mutant == "first_pick_uniform" else wv, draws[0])
        D2 = orc.sq_dist_sequential(X, X[picks[0]])
        for k in range(1, K):
            picks[k] = real_pick(D2 if mutant == "seed_ignores_weight" else wv * D2, draws[k])
            D2 = np.minimum(D2, orc.sq_dist_sequential(X, X[picks[k]]))
        return picks

    def lloyd_mut(X, centers, n_iter, bf16_assign=True, w=None):
        if w is None:
            return real_lloyd(X, centers, n_iter, bf16_assign)
        C = np.array(centers, dtype=np.float64)
        for _ in range(n_iter):
            A = orc.round_bf16(C) if bf16_assign else C
            assign = orc.nearest_codeword(X, A).idx
            new = C.copy()
            for k in range(C.shape[0]):
                m = np.flatnonzero(assign == k)
                if len(m):
                    new[k] = (w[m, None] * X[m]).sum(0) / len(m)
            C = new
        return C

    if mutant == "mean_over_count":
        monkeypatch.setattr(orc, "lloyd", lloyd_mut)
    else:
        monkeypatch.setattr(orc, "kmeanspp_seed", seed_mut)
    failed = 0
    for chk in (test_weighted_lloyd_matches_scikit_learn, test_integer_weights_equal_duplicated_samples,
                test_zero_weight_outliers_change_nothing):
        try:
            chk()
        except AssertionError:
            failed += 1
    assert failed >= 1, f"mutant {mutant} not caught"
