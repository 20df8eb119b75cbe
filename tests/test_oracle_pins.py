"""Pins of the float64 oracle to facts fixed outside itself: closed forms,
invariants, special cases that reduce to library routines, brute force.

Each test names the mistake it is there to catch.
"""
import os

import numpy as np
import pytest
import scipy.cluster.vq as scvq
from scipy.special import logsumexp

import synth
from cachebuild import build_cache
from oracle import lvq_oracle as orc


# ----------------------------------------------------------------------------
# helpers: a textbook attention built from library routines only
# ----------------------------------------------------------------------------
def textbook_attention(q, K, V, pos_q, pos_k, base, scale):
    """RoPE via transformers' LLaMA rotate-half implementation, attention via torch SDPA (float64)."""
    import torch
    from transformers.models.llama.modeling_llama import apply_rotary_pos_emb
    d = q.shape[-1]
    inv = 1.0 / (base ** (torch.arange(0, d, 2, dtype=torch.float64) / d))

    def cos_sin(p):
        ang = torch.as_tensor(p, dtype=torch.float64)[:, None] * inv[None, :]
        emb = torch.cat([ang, ang], dim=-1)
        return emb.cos()[None], emb.sin()[None]

    qt = torch.as_tensor(q, dtype=torch.float64)[None, None, None, :]
    kt = torch.as_tensor(K, dtype=torch.float64)[None, None]
    vt = torch.as_tensor(V, dtype=torch.float64)[None, None]
    cq, sq = cos_sin([pos_q])
    ck, sk = cos_sin(pos_k)
    qr, _ = apply_rotary_pos_emb(qt, qt, cq, sq)
    kr, _ = apply_rotary_pos_emb(kt, kt, ck, sk)
    out = torch.nn.functional.scaled_dot_product_attention(qr, kr, vt, scale=scale)
    s = (kr[0, 0] @ qr[0, 0, 0]).numpy() * scale
    return out[0, 0, 0].numpy(), logsumexp(s), s


# ----------------------------------------------------------------------------
# P1: bit budget
# ----------------------------------------------------------------------------
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden_rows(name):
    """The data lines of a fixture under tests/golden (comments start with '#')."""
    with open(os.path.join(GOLDEN, name)) as f:
        return [line.split() for line in f if line.strip() and not line.startswith("#")]


BIT_RATES = {int(g): float(bpe) for _, g, bpe in golden_rows("bit_rates.txt")}


@pytest.mark.parametrize("Tc,G", [(1, 16), (2, 16), (4, 32), (1, 32), (2, 32), (4, 16)])
def test_p1_bits_per_element_independent_of_Tc(Tc, G):
    """One byte per (block, head, group, K/V): the pages' 0.5 (G = 16) and 0.25 (G = 32)
    bits per element whatever Tc is.  Catches a layout that stores one row per step
    instead of one per block."""
    T, H, d = 8, 4, 128
    nbytes = orc.index_bytes_per_token(T, Tc, G, H, d)
    assert nbytes * 8 / (2 * T * H * d) == pytest.approx(BIT_RATES[G])
    # and the encoder's own output has exactly that many bytes per token
    rng = np.random.default_rng(1)
    kv = synth.f32_to_bf16_bits(rng.standard_normal((T, 3, H, d)))
    cb = synth.random_codebooks(rng, T, Tc, G, H, d)
    r = orc.encode(kv, cb, 0, T, Tc, G)
    assert r.idx[:, 0].size * 2 == nbytes


def test_divisibility_rule():
    with pytest.raises(ValueError):
        orc.check_divisibility(4, 3, 12, 64)      # Tc does not divide T
    with pytest.raises(ValueError):
        orc.check_divisibility(4, 4, 30, 64)      # Tc does not divide G
    with pytest.raises(ValueError):
        orc.check_divisibility(4, 2, 12, 64)      # c = 6 does not tile d = 64
    orc.check_divisibility(4, 2, 16, 64)


# ----------------------------------------------------------------------------
# P9 / P11: nearest codeword against brute force and a library VQ routine
# ----------------------------------------------------------------------------
def test_p9_nearest_matches_scipy_vq():
    """scipy.cluster.vq.vq is an independent nearest-code routine.
    Catches a wrong distance (dropped term, wrong sign) or a wrong axis."""
    rng = np.random.default_rng(2)
    for G in (8, 16, 32):
        C = rng.standard_normal((256, G))
        x = rng.standard_normal((700, G)) * 1.3
        r = orc.nearest_codeword(x, C)
        ref, dist = scvq.vq(x, C, check_finite=False)
        amb = r.n_near > 1
        assert amb.sum() < 3
        np.testing.assert_array_equal(r.idx[~amb], ref[~amb])
        np.testing.assert_allclose(r.d1, dist ** 2, rtol=1e-10)
        D = ((x[:, None, :] - C[None]) ** 2).sum(-1)
        assert np.all(r.d1[:, None] <= D + 1e-12)
        assert np.all(r.d2 >= r.d1)


def test_p9_tiny_hand_cases():
    """Hand-checkable 2-D cases, including an exact four-way tie (lowest index wins)."""
    C = np.array([[0, 0], [1, 0], [0, 1], [1, 1], [2, 2]], dtype=np.float64)
    x = np.array([[0.9, 0.1], [0.5, 0.5], [1.6, 1.6], [1.0, 1.0], [-3, 0.2]])
    r = orc.nearest_codeword(x, C)
    np.testing.assert_array_equal(r.idx, [1, 0, 4, 3, 0])
    np.testing.assert_allclose(r.d1, [0.02, 0.5, 0.32, 0.0, 9.04])
    np.testing.assert_array_equal(r.n_near[:4], [1, 4, 1, 1])


def test_p11_duplicate_codewords_lowest_index():
    """Repeated codewords return the lowest index.  Catches argmax-style last-index ties."""
    rng = np.random.default_rng(3)
    C = rng.standard_normal((256, 16))
    C[200] = C[17]
    C[31] = C[17]
    x = C[17] + 1e-3 * rng.standard_normal((50, 16))
    r = orc.nearest_codeword(x, C)
    assert np.all(r.idx == 17)


# ----------------------------------------------------------------------------
# P3: product-codebook separability (Tc = 2)
# ----------------------------------------------------------------------------
def test_p3_product_codebook_separates():
    """With codeword 16a+b = (A_a for step 0, B_b for step 1) the joint squared distance is
    the sum of two per-step distances, so the joint argmin is (argmin_A, argmin_B).
    Catches a joint vector gathered in the wrong element order or from the wrong steps."""
    rng = np.random.default_rng(4)
    T, Tc, G, H, d, N = 4, 2, 16, 2, 32, 300
    c = G // Tc
    nblk, ng = T // Tc, d // c
    cb = np.zeros((nblk, 2, H, ng, Tc, 256, c), dtype=np.float32)
    A = rng.standard_normal((nblk, 2, H, ng, 16, c)).astype(np.float32)
    Bb = rng.standard_normal((nblk, 2, H, ng, 16, c)).astype(np.float32)
    for a in range(16):
        for b in range(16):
            cb[:, :, :, :, 0, 16 * a + b] = A[:, :, :, :, a]
            cb[:, :, :, :, 1, 16 * a + b] = Bb[:, :, :, :, b]
    cbb = synth.f32_to_bf16_bits(cb)
    A64 = orc.bf16_to_f64(synth.f32_to_bf16_bits(A))
    B64 = orc.bf16_to_f64(synth.f32_to_bf16_bits(Bb))
    kv = synth.f32_to_bf16_bits(rng.standard_normal((T, N, H, d)))
    X = orc.bf16_to_f64(kv)
    for kv_sel in (0, 1):
        r = orc.encode(kv, cbb, kv_sel, T, Tc, G)
        for beta in range(nblk):
            for h in range(H):
                for g in range(ng):
                    xa = X[beta * Tc + 0, :, h, g * c:(g + 1) * c]
                    xb = X[beta * Tc + 1, :, h, g * c:(g + 1) * c]
                    ia, _ = scvq.vq(xa, A64[beta, kv_sel, h, g], check_finite=False)
                    ib, _ = scvq.vq(xb, B64[beta, kv_sel, h, g], check_finite=False)
                    ok = r.n_near[beta, :, h, g] == 1
                    np.testing.assert_array_equal(r.idx[beta, :, h, g][ok], (16 * ia + ib)[ok])


# ----------------------------------------------------------------------------
# P2: Tc = 1 is per-step coding
# ----------------------------------------------------------------------------
def test_p2_tc1_is_per_step_coding():
    """encode(X, Tc=1)[t] equals coding step t alone with its own books, and the decode
    attention at step t equals the attention of a one-step cache built from step t alone.
    Catches block/step index mix-ups."""
    T, Tc, G, H, d = 4, 1, 16, 1, 64
    cache = build_cache(11, 2, [45, 70], H, d, T, Tc, G, 4, 16, books="random", shuffle=True)
    for b in range(2):
        toks = cache.k_tokens[b][:, :int(cache.q_end[b])]
        full = orc.encode(toks, cache.codebooks, 0, T, Tc, G)
        for t in range(T):
            one = orc.encode(toks[t:t + 1], cache.codebooks[t:t + 1], 0, 1, 1, G)
            np.testing.assert_array_equal(full.idx[t], one.idx[0])
    for t in range(T):
        out, lse = cache.oracle_attn(t)
        # one-step cache: step t's tokens, step t's books, the same page placement
        ip1 = cache.index_pages[:, t:t + 1]
        bp1 = cache.bf16_pages[:, t:t + 1]
        shp1 = orc.AttnShape(cache.B, H, H, d, 1, 1, G, 4)
        o1, l1 = orc.decode_attn(shp1, cache.q[t], cache.page_table, ip1, bp1, cache.bf16_table,
                                 cache.codebooks[t:t + 1], 0, cache.pos, cache.seq_len, cache.q_end)
        np.testing.assert_array_equal(out, o1)
        np.testing.assert_array_equal(lse, l1)


# ----------------------------------------------------------------------------
# P4: all tokens bf16 = textbook RoPE + softmax attention
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("L,Hq", [(37, 4), (1, 2), (64, 2)])
def test_p4_all_bf16_is_textbook_attention(L, Hq):
    """q_end = 0: every token is bf16, so decode attention must equal RoPE (transformers'
    rotate-half implementation) + scaled dot-product attention (torch).  The queries sit at
    positions other than the lengths (13 beyond the first sequence, 3 inside the second:
    the position is an input of its own).  Catches a RoPE sign or pairing error, a wrong
    scale, a wrong GQA head map, a query rotated at the wrong position, a dropped sink or
    recent token."""
    H, d, T = 2, 64, 4
    cache = build_cache(12, 2, [L, L + 5], H, d, T, 2, 16, 4, 16, Hq=Hq, books="random",
                        q_end=[0, 0])
    cache.pos = np.array([L + 13, 3])
    for t in (0, 3):
        out, lse = cache.oracle_attn(t)
        for b in range(2):
            Lb = int(cache.seq_len[b])
            for hq in range(Hq):
                h = hq // (Hq // H)
                K = orc.bf16_to_f64(cache.k_tokens[b][t, :, h])
                V = orc.bf16_to_f64(cache.v_tokens[b][t, :, h])
                q = orc.bf16_to_f64(cache.q[t, b, hq])
                o_ref, l_ref, _ = textbook_attention(q, K, V, int(cache.pos[b]), np.arange(Lb),
                                                     10000.0, 1 / np.sqrt(d))
                np.testing.assert_allclose(out[b, hq], o_ref, rtol=1e-10, atol=1e-12)
                np.testing.assert_allclose(lse[b, hq], l_ref, rtol=1e-12)


# ----------------------------------------------------------------------------
# P5: identity codebook makes the coded cache exact
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("Tc,G", [(2, 16), (4, 32), (1, 32)])
def test_p5_identity_codebook_end_to_end(Tc, G):
    """Key codeword k = joint vector of key token k, value codeword qe - 1 - k = joint vector
    of value token k (so the K and V index rows differ), every distance to the right
    codeword is 0, the indices are known, and the coded cache reproduces the bf16 tokens
    exactly: coded attention must equal textbook attention on the raw tokens.  Catches any
    layout error in gather, encode, page scatter (K and V halves included), index-row read,
    step-slice read or value reconstruction."""
    T, H, d, L, n_sink, n_recent = 4, 2, 64, 61, 4, 16
    cache = build_cache(13, 1, [L], H, d, T, Tc, G, n_sink, n_recent, books="random",
                        index="random", shuffle=True)
    c = G // Tc
    nblk, ng = T // Tc, d // c
    qe = int(cache.q_end[0])
    assert qe == 40
    X = {0: orc.bf16_to_f64(cache.k_tokens[0]), 1: orc.bf16_to_f64(cache.v_tokens[0])}
    cb = orc.bf16_to_f64(cache.codebooks).copy()
    rng = np.random.default_rng(5)
    cb[...] = 50.0 + rng.standard_normal(cb.shape)            # far-away filler codewords
    order = {0: np.arange(qe), 1: np.arange(qe)[::-1]}        # codeword of token k
    for kv in (0, 1):
        for beta in range(nblk):
            for tau in range(Tc):
                for g in range(ng):
                    cb[beta, kv, :, g, tau][:, order[kv], :] = X[kv][beta * Tc + tau, :qe, :, g * c:(g + 1) * c].transpose(1, 0, 2)
    cbb = synth.f32_to_bf16_bits(cb.astype(np.float32))
    assert np.array_equal(orc.bf16_to_f64(cbb)[..., :qe, :], cb[..., :qe, :])
    ip = np.zeros_like(cache.index_pages)
    for kv in (0, 1):
        toks = cache.k_tokens[0] if kv == 0 else cache.v_tokens[0]
        r = orc.encode(toks[:, :qe], cbb, kv, T, Tc, G)
        expect = np.broadcast_to(order[kv][None, :, None, None], r.idx.shape)
        np.testing.assert_array_equal(r.idx, expect)
        assert np.all(r.d1 == 0)
        orc.scatter_index_pages(r.idx, kv, cache.page_table[0, :qe // 8], ip)
    shp = cache.shape()
    for t in range(T):
        out, lse = orc.decode_attn(shp, cache.q[t], cache.page_table, ip, cache.bf16_pages,
                                   cache.bf16_table, cbb, t, cache.pos, cache.seq_len, cache.q_end)
        for h in range(H):
            o_ref, l_ref, _ = textbook_attention(orc.bf16_to_f64(cache.q[t, 0, h]), X[0][t, :, h],
                                                 X[1][t, :, h], L, np.arange(L), 10000.0, 1 / np.sqrt(d))
            np.testing.assert_allclose(out[0, h], o_ref, rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(lse[0, h], l_ref, rtol=1e-12)


# ----------------------------------------------------------------------------
# P6: split + log-sum-exp merge = unsplit
# ----------------------------------------------------------------------------
def test_p6_lse_merge_equals_unsplit():
    """Flash-Decoding splits merged by log-sum-exp give the unsplit result for any partition.
    Catches a wrong rescale factor or a lost chunk in the merge."""
    cache = build_cache(14, 2, [97, 130], 1, 64, 4, 2, 16, 4, 16, books="random", index="random")
    shp = cache.shape()
    for t in (1, 2):
        ref, lref = cache.oracle_attn(t)
        n_pages = int(max(cache.q_end)) // 8
        for S in (1, 2, 7, n_pages):
            o, l = orc.decode_attn_split(shp, cache.q[t], cache.page_table, cache.index_pages,
                                         cache.bf16_pages, cache.bf16_table, cache.codebooks, t,
                                         cache.pos, cache.seq_len, cache.q_end, S)
            np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(l, lref, rtol=1e-13)
    # the merge itself against scipy's logsumexp
    rng = np.random.default_rng(6)
    s = rng.standard_normal(50) * 5
    v = rng.standard_normal((50, 3))
    parts = []
    for lo, hi in ((0, 10), (10, 10), (10, 33), (33, 50)):
        if hi > lo:
            m = s[lo:hi].max()
            w = np.exp(s[lo:hi] - m)
            parts.append((m, w.sum(), w @ v[lo:hi]))
        else:
            parts.append((-np.inf, 0.0, np.zeros(3)))
    o, l = orc.lse_merge(parts)
    assert l == pytest.approx(logsumexp(s), rel=1e-14)
    np.testing.assert_allclose(o, np.exp(s - logsumexp(s)) @ v, rtol=1e-12)


# ----------------------------------------------------------------------------
# P7: only the step-t slice is read
# ----------------------------------------------------------------------------
def test_p7_step_slice_locality():
    """Perturbing codebook slices of other steps (tau' != t % Tc) or other blocks
    (beta' != t // Tc) leaves the step-t output bit-identical.  Catches reading the wrong slice."""
    T, Tc, G = 4, 2, 16
    cache = build_cache(15, 1, [150], 2, 64, T, Tc, G, 4, 16, books="random", index="random")
    rng = np.random.default_rng(7)
    for t in range(T):
        beta, tau = t // Tc, t % Tc
        ref = cache.oracle_attn(t)
        cb = cache.codebooks.copy()
        noise = rng.integers(0, 1 << 16, size=cb.shape, dtype=np.uint16) & np.uint16(0x3FFF)
        mask = np.ones(cb.shape, dtype=bool)
        mask[beta, :, :, :, tau] = False
        cb[mask] = noise[mask]
        alt = orc.decode_attn(cache.shape(), cache.q[t], cache.page_table, cache.index_pages,
                              cache.bf16_pages, cache.bf16_table, cb, t, cache.pos,
                              cache.seq_len, cache.q_end)
        np.testing.assert_array_equal(ref[0], alt[0])
        np.testing.assert_array_equal(ref[1], alt[1])
        # and the slice that is read does matter
        cb2 = cache.codebooks.copy()
        cb2[beta, :, :, :, tau] ^= np.uint16(0x0040)
        alt2 = orc.decode_attn(cache.shape(), cache.q[t], cache.page_table, cache.index_pages,
                               cache.bf16_pages, cache.bf16_table, cb2, t, cache.pos,
                               cache.seq_len, cache.q_end)
        assert not np.allclose(ref[0], alt2[0])


# ----------------------------------------------------------------------------
# P8: physical page placement does not matter
# ----------------------------------------------------------------------------
def test_p8_page_permutation_invariance():
    """The same cache placed in a shuffled and in an identity page pool gives identical output.
    Catches indexing pages by logical instead of physical id."""
    kw = dict(books="random", index="oracle")
    a = build_cache(16, 2, [90, 123], 1, 64, 4, 2, 16, 4, 16, shuffle=True, **kw)
    b = build_cache(16, 2, [90, 123], 1, 64, 4, 2, 16, 4, 16, shuffle=False, **kw)
    assert not np.array_equal(a.page_table, b.page_table)
    for t in range(4):
        oa, la = a.oracle_attn(t)
        ob, lb = b.oracle_attn(t)
        np.testing.assert_array_equal(oa, ob)
        np.testing.assert_array_equal(la, lb)


# ----------------------------------------------------------------------------
# P10: RoPE closed forms and relative-position invariance
# ----------------------------------------------------------------------------
def test_p10_rope_relative_invariance_and_closed_forms():
    """Scores depend only on p - pos (checked up to 64K), the rotation keeps norms, and the
    d = 2 case is a plain rotation by p radians.  Catches phase or frequency mistakes."""
    rng = np.random.default_rng(8)
    d = 128
    q = rng.standard_normal(d)
    K = rng.standard_normal((40, d))
    p = rng.integers(0, 60000, size=40)
    for delta in (1, 777, 65536):
        s0 = orc.rope(K, p) @ orc.rope(q, 1000)
        s1 = orc.rope(K, p + delta) @ orc.rope(q, 1000 + delta)
        np.testing.assert_allclose(s0, s1, rtol=1e-9, atol=1e-9)
    np.testing.assert_allclose(np.linalg.norm(orc.rope(K, p), axis=1), np.linalg.norm(K, axis=1))
    np.testing.assert_array_equal(orc.rope(K, np.zeros(40)), K)
    x = np.array([1.0, 0.0])
    for pp in (0, 1, 2.5):
        np.testing.assert_allclose(orc.rope(x, pp), [np.cos(pp), np.sin(pp)], atol=1e-15)
    th = orc.rope_inv_freq(8)
    np.testing.assert_allclose(th, [1.0, 10000 ** -0.25, 10000 ** -0.5, 10000 ** -0.75])


# ----------------------------------------------------------------------------
# P12 and boundary conventions
# ----------------------------------------------------------------------------
def test_p12_single_token():
    """L = 1: the only weight is 1, so out = v_0 and lse = s_0."""
    cache = build_cache(17, 2, [1, 1], 2, 64, 4, 2, 16, 4, 16, books="random", q_end=[0, 0])
    for t in range(4):
        out, lse, sc = cache.oracle_attn(t, return_scores=True)
        for b in range(2):
            for h in range(2):
                np.testing.assert_array_equal(out[b, h], orc.bf16_to_f64(cache.v_tokens[b][t, 0, h]))
                assert lse[b, h] == sc[(b, h)][0]


def test_p13_empty_sequence_is_the_merge_identity():
    """L = 0 (an empty batch slot): out = 0 and lse = -inf, the partial that the
    log-sum-exp merge leaves every other partial unchanged with (scipy's logsumexp of
    [x, -inf] is x), and an empty slot changes no other sequence's result."""
    with_empty = build_cache(37, 3, [0, 45, 0], 2, 128, 4, 4, 32, 4, 16, books="random", index="random")
    out, lse = with_empty.oracle_attn(1)
    for b in (0, 2):
        np.testing.assert_array_equal(out[b], 0.0)
        assert np.isneginf(lse[b]).all()
    assert np.isfinite(lse[1]).all()
    for h in range(2):
        assert logsumexp([lse[1, h], lse[0, h]]) == pytest.approx(lse[1, h], abs=0, rel=1e-15)
    # the same sequence alone, same inputs: only slot 1 of the batch above
    c = with_empty
    alone = orc.decode_attn(orc.AttnShape(1, 2, 2, 128, 4, 4, 32, 4), c.q[1][1:2], c.page_table[1:2],
                            c.index_pages, c.bf16_pages, c.bf16_table[1:2], c.codebooks, 1,
                            c.pos[1:2], c.seq_len[1:2], c.q_end[1:2])
    np.testing.assert_array_equal(alone[0][0], out[1])
    np.testing.assert_array_equal(alone[1][0], lse[1])


def test_boundary_conventions():
    """First 4 and last 16 of 512 tokens bf16 leaves 492 coded tokens; sink wins over recent."""
    assert synth.prefill_q_end(512, 16) == 496
    cls = orc.token_classes(512, 496, 4)
    assert (cls == 1).sum() == 492 and (cls == 0).sum() == 4 and (cls == 2).sum() == 16
    cls = orc.token_classes(20, 0, 4)
    assert (cls == 0).sum() == 4 and (cls == 2).sum() == 16
    assert synth.prefill_q_end(10, 16) == 0
    assert synth.prefill_q_end(32768, 64) == 32704


# ----------------------------------------------------------------------------
# P14: attention mass of a span of positions (the needle check)
# ----------------------------------------------------------------------------
def test_p14_needle_mass():
    """needle_mass(s, lse, lo, hi) is the softmax mass of positions [lo, hi): it equals
    scipy's softmax summed over the span, the whole range has mass 1, disjoint spans add,
    an empty span has mass 0, and a hand case: scores (0, ln 3) give the second position
    3/4 of the mass."""
    from scipy.special import softmax
    rng = np.random.default_rng(14)
    s = rng.standard_normal(300) * 4.0
    s[120:136] += 9.0                                   # a needle span that dominates
    lse = float(logsumexp(s))
    for lo, hi in ((120, 136), (0, 300), (0, 1), (299, 300), (7, 200)):
        assert orc.needle_mass(s, lse, lo, hi) == pytest.approx(softmax(s)[lo:hi].sum(), rel=1e-12, abs=1e-15)
    assert orc.needle_mass(s, lse, 0, 300) == pytest.approx(1.0, rel=1e-13)
    assert orc.needle_mass(s, lse, 0, 50) + orc.needle_mass(s, lse, 50, 300) == pytest.approx(1.0, rel=1e-13)
    assert orc.needle_mass(s, lse, 40, 40) == 0.0
    hand = np.array([0.0, np.log(3.0)])
    assert orc.needle_mass(hand, np.log(4.0), 1, 2) == pytest.approx(0.75, rel=1e-15)
    assert orc.needle_mass(hand, np.log(4.0), 0, 1) == pytest.approx(0.25, rel=1e-15)
    # with the oracle's own scores and lse of a planted span: the same as scipy on those scores
    cache = build_cache(18, 1, [260], 1, 64, 4, 2, 16, 4, 16, books="random", index="random")
    out, lse_o, sc = cache.oracle_attn(2, return_scores=True)
    scores = sc[(0, 0)]
    assert lse_o[0, 0] == pytest.approx(logsumexp(scores), rel=1e-14)
    assert orc.needle_mass(scores, lse_o[0, 0], 30, 46) == pytest.approx(softmax(scores)[30:46].sum(), rel=1e-12)
