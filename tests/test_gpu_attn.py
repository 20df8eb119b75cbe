"""GPU decode-attention parity against the float64 oracle, through the C ABI.

Tolerance: max-abs <= 2e-3 over every output element and max-rel <= 1e-2 over
the elements with |oracle| >= 0.2, on the float32 output; lse within 1e-4
absolute.  Full context lengths run on the GPU in the launch configuration the
benchmark uses; the oracle checks every (sequence, head) pair of the Ouro-shaped
call and every head of the 64K needle call.  Each case's figures go to the
parity record (parity_log).
"""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from cachebuild import build_cache, build_cache_light
from gpu_helpers import attn_close, gpu_attn, to_dev
from oracle import lvq_oracle as orc
import parity_log as plog

pytestmark = pytest.mark.gpu


def check(out, lse, ref_out, ref_lse, label, pairs=None):
    o = out.cpu().numpy()
    l = lse.cpu().numpy()
    if pairs is not None:
        o = np.stack([o[b, h] for b, h in pairs])
        l = np.array([l[b, h] for b, h in pairs])
        ref_out = np.stack([ref_out[b, h] for b, h in pairs])
        ref_lse = np.array([ref_lse[b, h] for b, h in pairs])
    ok, mabs, mrel = attn_close(o, ref_out)
    # an empty sequence has lse = -inf on both sides; the rest must be finite and close
    empty = np.isneginf(ref_lse)
    np.testing.assert_array_equal(np.isneginf(l), empty, err_msg=f"{label}: -inf lse pattern")
    lerr = float(np.abs(l[~empty] - ref_lse[~empty]).max()) if (~empty).any() else 0.0
    n_rows = int(np.prod(o.shape[:-1]))
    plog.line(f"{label}: {n_rows} (b, head) rows x {o.shape[-1]} channels, max-abs {mabs:.3e}, "
              f"max-rel {mrel:.3e} (|ref| >= 0.2), lse max-abs {lerr:.3e}")
    assert ok, f"{label}: output outside tolerance (max-abs {mabs:.3e}, max-rel {mrel:.3e})"
    assert lerr <= 1e-4, f"{label}: lse error {lerr:.3e}"


def test_tiny_config_all_steps():
    """The tiny configuration end to end: oracle-encoded pages, k-means books, every step."""
    plog.case("attention, tiny configuration: d=64 H=1 T=4 Tc=2 G=16 L=512, k-means books on 4096 samples")
    cache = build_cache(1, 1, [512], 1, 64, 4, 2, 16, 4, 16, book_samples=4096)
    dc = to_dev(cache)
    for t in range(4):
        out, lse = gpu_attn(dc, t)
        ro, rl = cache.oracle_attn(t)
        check(out, lse, ro, rl, f"t={t}")


EDGE = [  # config, B, lengths, H, Hq, d, T, Tc, G, n_sink, n_recent
    (31, 2, [37, 70], 2, 4, 64, 4, 2, 16, 4, 16),        # GQA, ragged lengths
    (32, 3, [1, 8, 19], 1, 1, 128, 4, 4, 32, 4, 64),      # shorter than sink + recent: all bf16
    (33, 2, [300, 129], 2, 2, 128, 8, 4, 32, 4, 64),      # two loop blocks
    (34, 1, [1000], 2, 2, 128, 1, 1, 32, 4, 64),          # prelude layer: Tc=1, c=32
    (35, 2, [515, 260], 1, 2, 128, 4, 2, 32, 0, 16),      # c = 16, no sink
    (36, 1, [600], 1, 1, 64, 4, 4, 32, 8, 8),             # d = 64, n_sink = 8, c = 8
    (37, 3, [0, 45, 0], 2, 2, 128, 4, 4, 32, 4, 16),      # empty batch slots: out 0, lse -inf
    (38, 3, [45, 0, 20], 1, 16, 128, 4, 4, 32, 4, 16),    # the same on the multi-row route (GQA 16)
    (72, 3, [45, 0, 20], 1, 4, 128, 4, 4, 32, 4, 16),     # the same on the grouped route (GQA 4)
    (73, 3, [45, 0, 20], 1, 8, 128, 4, 4, 32, 4, 16),     # the same on the multi-row route at GQA 8
    (74, 2, [200, 333], 2, 2, 64, 4, 2, 32, 4, 16),       # d = 64 with c = 16
    (75, 2, [129, 64], 2, 4, 128, 4, 4, 32, 4, 16),       # grouped route at GQA 2, ragged
    (76, 3, [72, 79, 80], 2, 2, 128, 4, 4, 32, 4, 64),    # q_end = 8, 8, 16: coded tokens 4..7 share page 0 with the sink
    (77, 2, [72, 80], 1, 16, 128, 4, 4, 32, 8, 64),       # n_sink = 8 = q_end: an empty coded range, multi-row route
    (82, 2, [333, 90], 2, 6, 128, 4, 4, 32, 4, 16),       # 3 query heads per KV head: the per-head kernel's GQA map
    (83, 2, [333, 90], 1, 12, 128, 4, 2, 32, 4, 16),      # 12 per KV head: multi-row route, 4 padding rows
]


@pytest.mark.parametrize("cfg,B,lengths,H,Hq,d,T,Tc,G,ns,nr", EDGE)
def test_edge_cases(cfg, B, lengths, H, Hq, d, T, Tc, G, ns, nr):
    plog.case(f"attention edge case cfg={cfg} B={B} L={lengths} H={H} Hq={Hq} d={d} T={T} Tc={Tc} G={G} "
              f"n_sink={ns} n_recent={nr}")
    cache = build_cache(cfg, B, lengths, H, d, T, Tc, G, ns, nr, Hq=Hq, books="random",
                        index="random")
    dc = to_dev(cache)
    for t in sorted({0, T - 1}):
        out, lse = gpu_attn(dc, t)
        ro, rl = cache.oracle_attn(t)
        check(out, lse, ro, rl, f"t={t}")


def test_split_counts_and_page_permutation():
    """Splits 1, 2, 7 and one per tile agree with the oracle and with each other; a page
    table over an identity pool gives the same bits as the shuffled one."""
    plog.case("attention split counts 1/2/7/1000 and page permutation, B=2 L=[2000, 1111]")
    kw = dict(books="random", index="oracle")
    cache = build_cache(37, 2, [2000, 1111], 2, 128, 4, 4, 32, 4, 64, **kw)
    dc = to_dev(cache)
    t = 2
    ro, rl = cache.oracle_attn(t)
    outs = []
    for S in (1, 2, 7, 1000):
        out, lse = gpu_attn(dc, t, n_splits=S)
        check(out, lse, ro, rl, f"splits={S}")
        outs.append(out.cpu().numpy())
    for o in outs[1:]:
        np.testing.assert_allclose(o, outs[0], rtol=2e-5, atol=2e-6)
    flat = build_cache(37, 2, [2000, 1111], 2, 128, 4, 4, 32, 4, 64, shuffle=False, **kw)
    o1, _ = gpu_attn(to_dev(flat), t, n_splits=7)
    o2, _ = gpu_attn(dc, t, n_splits=7)
    np.testing.assert_array_equal(o1.cpu().numpy(), o2.cpu().numpy())
    # same inputs twice: identical bits
    o3, _ = gpu_attn(dc, t, n_splits=7)
    np.testing.assert_array_equal(o3.cpu().numpy(), o2.cpu().numpy())


def test_many_sequences_token_balanced_split():
    """70 sequences (more than one 64-lane scan block) with lengths U[1, 400] and GQA 2:
    every (b, head) against the oracle for automatic, one-workgroup and 1008-wave splits
    (the last leaves most waves with empty ranges); the three agree closely."""
    plog.case("attention token-balanced split, B=70 lengths U[1,400], GQA 2, splits 0/1/1000")
    rl_ = np.random.default_rng(synth.seed_for(40, synth.STREAM_LENGTHS))
    lengths = synth.uniform_lengths(rl_, 70, 1, 400)
    cache = build_cache(40, 70, lengths, 2, 128, 4, 4, 32, 4, 16, Hq=4, books="random", index="random")
    dc = to_dev(cache)
    t = 3
    ro, rl = cache.oracle_attn(t)
    outs = []
    for S in (0, 1, 1000):
        out, lse = gpu_attn(dc, t, n_splits=S)
        check(out, lse, ro, rl, f"splits={S}")
        outs.append(out.cpu().numpy())
    for o in outs[1:]:
        np.testing.assert_allclose(o, outs[0], rtol=2e-5, atol=2e-6)


@pytest.mark.parametrize("route,H,Hq", [("per-head", 2, 2), ("multi-row", 1, 16)])
def test_index_pool_beyond_4gib(route, H, Hq):
    """An index pool over 4 GiB takes the kernels' 64-bit page addressing.  The same pages
    moved to the top of such a pool give the same bits as the compact pool (page
    placement invariance), so the 32-bit and 64-bit address paths agree."""
    plog.case(f"attention, index pool over 4 GiB (64-bit page addressing), {route} route: "
              f"bit-identical to the compact pool")
    cache = build_cache(39, 1, [2000], H, 128, 4, 4, 32, 4, 64, Hq=Hq, books="random", index="random")
    dc = to_dev(cache)
    ref, ref_lse = gpu_attn(dc, 1)
    pool = dc.index_pages
    page_bytes = pool[0].numel()
    n_big = (4 << 30) // page_bytes + 4096
    assert n_big * page_bytes > 1 << 32
    big = torch.empty((n_big,) + tuple(pool.shape[1:]), dtype=pool.dtype, device=pool.device)
    off = n_big - pool.shape[0]
    big[off:] = pool
    pt = dc.page_table.clone()
    pt[pt >= 0] += off
    got, got_lse = gpu_attn(dataclasses.replace(dc, index_pages=big, page_table=pt), 1)
    del big
    torch.cuda.empty_cache()
    np.testing.assert_array_equal(got.cpu().numpy(), ref.cpu().numpy())
    np.testing.assert_array_equal(got_lse.cpu().numpy(), ref_lse.cpu().numpy())


def test_step_slice_locality_on_gpu():
    """Changing codebook slices of other steps/blocks leaves the step-t output bit-identical."""
    cache = build_cache(38, 1, [700], 1, 128, 4, 2, 16, 4, 64, books="random", index="random")
    dc = to_dev(cache)
    for t in (1, 2):
        beta, tau = t // 2, t % 2
        o1, _ = gpu_attn(dc, t)
        cb = cache.codebooks.copy()
        mask = np.ones(cb.shape, bool)
        mask[beta, :, :, :, tau] = False
        cb[mask] ^= np.uint16(0x0101)
        dc.codebooks.copy_(torch.from_numpy(cb.view(np.int16)).cuda())
        o2, _ = gpu_attn(dc, t)
        dc.codebooks.copy_(torch.from_numpy(cache.codebooks.view(np.int16)).cuda())
        np.testing.assert_array_equal(o1.cpu().numpy(), o2.cpu().numpy())


ALL_PAIRS_C2 = [(b, h) for b in range(8) for h in range(16)]


def test_ouro_shape_full_context_all_pairs():
    """Ouro-1.4B-shaped call: B=8, 32768 tokens, 16 heads, d=128, T=4, Tc=4, G=32,
    4 sink + 64 recent, shuffled pages, in the benchmark's launch configuration.  The
    cache holds the generator's own tokens coded against k-means books (realistic codes
    and value scales); every (b, head) pair at every loop step is checked."""
    plog.case("attention, Ouro-shaped B=8 L=32768 H=16 d=128 T=4 Tc=4 G=32: generated tokens, "
              "k-means books (4096 samples), nearest-codeword indices; all 128 (b, head) pairs")
    from cachebuild import build_cache_generated
    cache = build_cache_generated(2, 8, [32768] * 8, 16, 128, 4, 4, 32, 4, 64)
    dc = to_dev(cache)
    for t in range(4):
        out, lse = gpu_attn(dc, t)
        ro, rl = orc.decode_attn(cache.shape(), cache.q[t], cache.page_table, cache.index_pages,
                                 cache.bf16_pages, cache.bf16_table, cache.codebooks, t, cache.pos,
                                 cache.seq_len, cache.q_end, pairs=ALL_PAIRS_C2)
        check(out, lse, ro, rl, f"t={t}", pairs=ALL_PAIRS_C2)


def test_ouro_shape_uniform_codes_all_pairs():
    """The same shape with uniform random codes over Gaussian books on the data's channel
    scales (every codeword equally likely, so every LDS gather pattern occurs); all 128
    (b, head) pairs at the first loop step."""
    plog.case("attention, Ouro-shaped B=8 L=32768: uniform random codes, Gaussian books; all 128 pairs")
    cache = build_cache_light(2, 8, [32768] * 8, 16, 128, 4, 4, 32, 4, 64, books="random")
    dc = to_dev(cache)
    t = 0
    out, lse = gpu_attn(dc, t)
    ro, rl = orc.decode_attn(cache.shape(), cache.q[t], cache.page_table, cache.index_pages,
                             cache.bf16_pages, cache.bf16_table, cache.codebooks, t, cache.pos,
                             cache.seq_len, cache.q_end, pairs=ALL_PAIRS_C2)
    check(out, lse, ro, rl, f"t={t}", pairs=ALL_PAIRS_C2)


def plant_needle(cache, lo, span, rng):
    """Plant a 16-token needle in sequence 0: the span's tokens share one code row per
    block, the codeword of largest norm (summed over the block's steps) in every group,
    and every loop step's query is reset so that, after RoPE, it has cosine 0.9 with
    that reconstructed key at the middle of the span (the rest of its direction is a
    seeded vector orthogonal to it) and scores 24 there."""
    T, Tc, G, H, d = cache.T, cache.Tc, cache.G, cache.H, cache.d
    c = G // Tc
    ng = d // c
    cb = orc.bf16_to_f64(cache.codebooks)                       # [nblk][2][H][ng][Tc][256][c]
    idx = np.argmax((cb[:, 0] ** 2).sum(axis=(3, 5)), axis=-1)  # [nblk][H][ng]
    for i in range(span):
        p = lo + i
        P = cache.page_table[0, p // 8]
        cache.index_pages[P, :, :, 0, p % 8, :] = idx
    pos = int(cache.pos[0])
    mid = lo + span // 2
    cos = 0.9
    for t in range(T):
        beta, tau = t // Tc, t % Tc
        for h in range(H):
            kh = np.concatenate([cb[beta, 0, h, g, tau, idx[beta, h, g]] for g in range(ng)])
            kr = orc.rope(kh, mid)
            kr /= np.linalg.norm(kr)
            u = rng.standard_normal(d)
            u -= (u @ kr) * kr
            u /= np.linalg.norm(u)
            qn = 24.0 * np.sqrt(d) / (cos * np.linalg.norm(kh))
            qr = qn * (cos * kr + np.sqrt(1.0 - cos * cos) * u)
            cache.q[t, 0, h] = synth.f32_to_bf16_bits(orc.rope(qr, -pos).astype(np.float32))


def test_needle_64k():
    """Long-context retrieval shape: B=1, 65536 tokens, 16 heads, T=4, Tc=2, G=16, split-K
    over the coded tokens; every head at every loop step: output, lse, every score and the
    needle's attention mass against the oracle."""
    plog.case("attention, 64K needle B=1 L=65536 H=16 d=128 T=4 Tc=2 G=16: all 16 heads, all 4 steps")
    cache = build_cache_light(3, 1, [65536], 16, 128, 4, 2, 16, 4, 64, books="kmeans",
                              book_samples=1024)
    rng = np.random.default_rng(synth.seed_for(3, synth.STREAM_NEEDLE))
    lo = int(rng.integers(1000, 60000)) // 8 * 8
    plant_needle(cache, lo, 16, rng)
    dc = to_dev(cache)
    heads = list(range(16))
    pairs = [(0, h) for h in heads]
    for t in range(4):
        out, lse, sc = gpu_attn(dc, t, scores=True)
        ro, rl, rs = orc.decode_attn(cache.shape(), cache.q[t], cache.page_table, cache.index_pages,
                                     cache.bf16_pages, cache.bf16_table, cache.codebooks, t,
                                     cache.pos, cache.seq_len, cache.q_end, return_scores=True,
                                     pairs=pairs)
        check(out, lse, ro, rl, f"t={t}", pairs=pairs)
        s = sc.cpu().numpy()
        l = lse.cpu().numpy()
        worst_mass, worst_score = 0.0, 0.0
        for h in heads:
            m_gpu = float(np.exp(s[0, h, lo:lo + 16].astype(np.float64) - l[0, h]).sum())
            m_ref = orc.needle_mass(rs[(0, h)], rl[0, h], lo, lo + 16)
            assert m_ref > 0.5          # the needle dominates (uniform mass would be 2.4e-4)
            assert abs(m_gpu - m_ref) <= 2e-3, f"t={t} h={h}: needle mass gpu {m_gpu} oracle {m_ref}"
            np.testing.assert_allclose(s[0, h], rs[(0, h)], atol=2e-3, rtol=1e-4)
            worst_mass = max(worst_mass, abs(m_gpu - m_ref))
            worst_score = max(worst_score, float(np.abs(s[0, h] - rs[(0, h)]).max()))
            if h in (0, 15):
                plog.line(f"t={t} h={h}: needle mass gpu {m_gpu:.6f} oracle {m_ref:.6f}")
        plog.line(f"t={t}: 16 heads, needle mass max |gpu - oracle| {worst_mass:.3e}, "
                  f"65536 scores per head max-abs {worst_score:.3e}")


def test_mixed_serving_batch_sampled():
    """Mixed batch: 64 sequences with lengths U[1024, 16384], T=8, Tc=4, G=32, plus the
    prelude layer coded per step (T=1, Tc=1, G=32); sampled (b, h) pairs."""
    plog.case("attention, mixed batch B=64 lengths U[1024,16384], looped T=8 Tc=4 G=32 and prelude "
              "T=1 Tc=1 G=32: 16 sampled (b, head) pairs per step")
    rl_ = np.random.default_rng(synth.seed_for(5, synth.STREAM_LENGTHS))
    lengths = synth.uniform_lengths(rl_, 64, 1024, 16384)
    prs = np.random.default_rng(55)
    pairs = [(int(b), int(h)) for b, h in zip(prs.integers(0, 64, 16), prs.integers(0, 16, 16))]
    for (T, Tc, G) in ((8, 4, 32), (1, 1, 32)):
        cache = build_cache_light(5, 64, lengths, 16, 128, T, Tc, G, 4, 64, books="random")
        dc = to_dev(cache)
        for t in sorted({0, T - 1}):
            out, lse = gpu_attn(dc, t)
            ro, rl = orc.decode_attn(cache.shape(), cache.q[t], cache.page_table, cache.index_pages,
                                     cache.bf16_pages, cache.bf16_table, cache.codebooks, t,
                                     cache.pos, cache.seq_len, cache.q_end, pairs=pairs)
            check(out, lse, ro, rl, f"T={T} t={t}", pairs=pairs)
        del dc
        torch.cuda.empty_cache()


@pytest.mark.parametrize("route,H,Hq", [("per-head", 2, 2), ("grouped", 2, 8), ("multi-row", 1, 16)])
def test_out_of_pool_page_ids_are_skipped_and_counted(route, H, Hq):
    """A coded page-table entry outside [0, n_index_pages) and a bf16-table entry outside
    [0, n_bf16_pages) are skipped by every decode route (their tokens are left out); with a
    counter in the shape each such lookup adds one to it.  On clean tables the counter stays
    0, and giving it never changes the output bits."""
    plog.case(f"out-of-pool page ids, {route} route (H={H}, Hq={Hq}): counted, skipped, output unchanged")
    cache = build_cache(85, 2, [300, 520], H, 128, 4, 4, 32, 4, 16, Hq=Hq, books="random", index="random")
    dc = to_dev(cache)
    t = 1
    counter = torch.zeros(1, dtype=torch.int32, device="cuda")
    clean, clean_lse = gpu_attn(dc, t)
    got, got_lse = gpu_attn(dc, t, rejected=counter)
    assert int(counter.item()) == 0
    np.testing.assert_array_equal(got.cpu().numpy(), clean.cpu().numpy())
    np.testing.assert_array_equal(got_lse.cpu().numpy(), clean_lse.cpu().numpy())
    ro, rl = cache.oracle_attn(t)
    check(got, got_lse, ro, rl, "clean tables")

    # sequence 1: coded pages 3..5 point past the pool; sequence 0: its first recent page is missing
    pt = dc.page_table.clone()
    pt[1, 3:6] = dc.index_pages.shape[0] + 7
    bt = dc.bf16_table.clone()
    bt[0, 1] = -1
    bad = dataclasses.replace(dc, page_table=pt, bf16_table=bt)
    plain, plain_lse = gpu_attn(bad, t)
    counter.zero_()
    got, got_lse = gpu_attn(bad, t, rejected=counter)
    n = int(counter.item())
    plog.line(f"planted: 3 coded pages of sequence 1, 1 recent bf16 page of sequence 0 -> {n} rejected lookups")
    assert n > 0
    np.testing.assert_array_equal(got.cpu().numpy(), plain.cpu().numpy())
    assert np.isfinite(got.cpu().numpy()).all()
    # the skipped coded pages of sequence 1 leave sequence 0's output as it was
    only1 = dataclasses.replace(dc, page_table=pt)
    o1, _ = gpu_attn(only1, t)
    np.testing.assert_array_equal(o1.cpu().numpy()[0], clean.cpu().numpy()[0])
    assert not np.array_equal(o1.cpu().numpy()[1], clean.cpu().numpy()[1])


@pytest.mark.parametrize("route,H,Hq", [("per-head", 2, 2), ("grouped", 2, 8), ("multi-row", 1, 16)])
def test_query_positions_other_than_the_length(route, H, Hq):
    """The query is rotated at pos[b], which the decode call takes as its own input: here
    one sequence at its length, one 500 positions beyond it and one at position 7, below
    most of its keys (attention is limited by seq_len only).  Each route must rotate the
    query at pos and each key at its own position."""
    plog.case(f"attention query positions other than the length, {route} route (H={H}, Hq={Hq})")
    lengths = [300, 261, 150]
    cache = build_cache(78, 3, lengths, H, 128, 4, 4, 32, 4, 16, Hq=Hq, books="random", index="random")
    cache.pos = np.asarray([300, 761, 7], dtype=np.int32)
    dc = to_dev(cache)
    for t in (0, 3):
        out, lse = gpu_attn(dc, t)
        ro, rl = cache.oracle_attn(t)
        check(out, lse, ro, rl, f"t={t}")
    # the same cache with pos = seq_len gives another result (the position is really used)
    base = dataclasses.replace(cache, pos=cache.seq_len.copy())
    ob, _ = gpu_attn(to_dev(base), 3)
    assert np.abs(ob.cpu().numpy()[1:] - out.cpu().numpy()[1:]).max() > 1e-3


@pytest.mark.parametrize("route,H,Hq", [("per-head", 2, 2), ("grouped", 2, 8), ("multi-row", 1, 16)])
def test_softmax_scale_and_rope_base(route, H, Hq):
    """A softmax scale other than 1/sqrt(d) (0.2, a sharper softmax) and RoPE tables built
    for base 500000 instead of 10000: both are inputs of the call, and each route must
    apply them as the oracle does."""
    plog.case(f"attention softmax scale 0.2 and RoPE base 500000, {route} route (H={H}, Hq={Hq})")
    cache = build_cache(79, 2, [700, 333], H, 128, 4, 4, 32, 4, 16, Hq=Hq, books="random", index="random")
    dc = to_dev(cache, rope_base=500000.0)
    for t in (1, 2):
        out, lse = gpu_attn(dc, t, scale=0.2)
        ro, rl = orc.decode_attn(dataclasses.replace(cache.shape(500000.0), scale=0.2), cache.q[t],
                                 cache.page_table, cache.index_pages, cache.bf16_pages, cache.bf16_table,
                                 cache.codebooks, t, cache.pos, cache.seq_len, cache.q_end)
        check(out, lse, ro, rl, f"t={t}")


@pytest.mark.parametrize("route,H,Hq", [("per-head", 2, 2), ("grouped", 2, 8), ("multi-row", 1, 16)])
def test_max_seq_len_far_above_the_lengths(route, H, Hq):
    """max_seq_len sizes the automatic split; here it is 40000 for sequences of 37 and 100
    tokens, so most waves get empty ranges and write no record (or records of weight 0)
    that the merge must ignore.  The result must not depend on it."""
    plog.case(f"attention with max_seq_len 40000 over lengths [37, 100], {route} route (H={H}, Hq={Hq})")
    cache = build_cache(80, 2, [37, 100], H, 128, 4, 4, 32, 4, 16, Hq=Hq, books="random", index="random")
    tight = to_dev(cache)
    loose = to_dev(cache, max_seq_len=40000)
    for t in (0, 3):
        out, lse = gpu_attn(loose, t)
        ro, rl = cache.oracle_attn(t)
        check(out, lse, ro, rl, f"t={t}")
        o2, l2 = gpu_attn(tight, t)
        np.testing.assert_allclose(out.cpu().numpy(), o2.cpu().numpy(), rtol=2e-5, atol=2e-6)


@pytest.mark.parametrize("route,H,Hq", [("per-head", 2, 2), ("grouped", 2, 8), ("multi-row", 1, 16)])
def test_three_hundred_short_sequences(route, H, Hq):
    """B = 300 sequences of 1 to 200 tokens (empty slots included): the work-list scan runs
    over five chunks of 64 sequences, and a wave's range meets many sequences, writing a
    record for each; every (sequence, head) against the oracle."""
    plog.case(f"attention over 300 short sequences, {route} route (H={H}, Hq={Hq})")
    rng = np.random.default_rng(81)
    lengths = rng.integers(1, 201, 300)
    lengths[[7, 150, 299]] = 0
    cache = build_cache(81, 300, lengths.tolist(), H, 128, 4, 4, 32, 4, 16, Hq=Hq, books="random",
                        index="random")
    dc = to_dev(cache)
    out, lse = gpu_attn(dc, 2)
    ro, rl = cache.oracle_attn(2)
    check(out, lse, ro, rl, "t=2")
