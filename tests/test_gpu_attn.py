"""GPU decode-attention parity against the float64 oracle, through the C ABI.

Tolerance (element-wise): |gpu - oracle| <= 2e-3 or <= 1e-2 * |oracle|, on the
float32 output; lse within 1e-4 absolute.  Full context lengths are run on the
GPU in the launch configuration the benchmark uses; the oracle checks sampled
(sequence, head) pairs.
"""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from cachebuild import build_cache, build_cache_light
from gpu_helpers import attn_close, gpu_attn, to_dev
from oracle import lvq_oracle as orc

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
    print(f"  {label}: max-abs {mabs:.2e} max-rel {mrel:.2e} lse err {lerr:.2e}", flush=True)
    assert ok, f"{label}: output outside tolerance (max-abs {mabs:.3e})"
    assert lerr <= 1e-4, f"{label}: lse error {lerr:.3e}"


def test_tiny_config_all_steps():
    """The tiny configuration end to end: oracle-encoded pages, k-means books, every step."""
    print("\ncase tiny d=64 H=1 T=4 Tc=2 G=16 L=512", flush=True)
    cache = build_cache(1, 1, [512], 1, 64, 4, 2, 16, 4, 16, book_samples=1024)
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
    (38, 3, [45, 0, 20], 1, 8, 128, 4, 4, 32, 4, 16),     # the same on the multi-row route (GQA 8)
]


@pytest.mark.parametrize("cfg,B,lengths,H,Hq,d,T,Tc,G,ns,nr", EDGE)
def test_edge_cases(cfg, B, lengths, H, Hq, d, T, Tc, G, ns, nr):
    print(f"\ncase edge cfg={cfg} B={B} L={lengths} H={H} Hq={Hq} d={d} T={T} Tc={Tc} G={G}", flush=True)
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
    print("\ncase splits / permutation", flush=True)
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
    print("\ncase B=70 lengths U[1,400] splits 0/1/1000", flush=True)
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


def test_index_pool_beyond_4gib():
    """An index pool over 4 GiB takes the kernel's 64-bit page addressing.  The same pages
    moved to the top of such a pool give the same bits as the compact pool (page
    placement invariance), so the 32-bit and 64-bit address paths agree."""
    print("\ncase index pool over 4 GiB", flush=True)
    cache = build_cache(39, 1, [2000], 2, 128, 4, 4, 32, 4, 64, books="random", index="random")
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


def test_ouro_shape_full_context_sampled():
    """Ouro-1.4B-shaped call: B=8, 32768 tokens, 16 heads, d=128, T=4, Tc=4, G=32,
    4 sink + 64 recent, shuffled pages; all heads on the GPU, 6 (b, h) pairs checked."""
    print("\ncase ouro-shaped B=8 L=32768", flush=True)
    cache = build_cache_light(2, 8, [32768] * 8, 16, 128, 4, 4, 32, 4, 64, books="random")
    dc = to_dev(cache)
    pairs = [(0, 0), (3, 7), (7, 15), (5, 2), (1, 11), (6, 9)]
    for t in (0, 3):
        out, lse = gpu_attn(dc, t)
        ro, rl = orc.decode_attn(cache.shape(), cache.q[t], cache.page_table, cache.index_pages,
                                 cache.bf16_pages, cache.bf16_table, cache.codebooks, t, cache.pos,
                                 cache.seq_len, cache.q_end, pairs=pairs)
        check(out, lse, ro, rl, f"t={t}", pairs=pairs)


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
    over the coded tokens; the needle's attention mass matches the oracle."""
    import sub_bit_loop_amd as lvq  # noqa: F401
    print("\ncase needle L=65536", flush=True)
    cache = build_cache_light(3, 1, [65536], 16, 128, 4, 2, 16, 4, 64, books="kmeans",
                              book_samples=1024)
    rng = np.random.default_rng(synth.seed_for(3, synth.STREAM_NEEDLE))
    lo = int(rng.integers(1000, 60000)) // 8 * 8
    plant_needle(cache, lo, 16, rng)
    dc = to_dev(cache)
    heads = [0, 5, 13]
    for t in (0, 3):
        out, lse, sc = gpu_attn(dc, t, scores=True)
        ro, rl, rs = orc.decode_attn(cache.shape(), cache.q[t], cache.page_table, cache.index_pages,
                                     cache.bf16_pages, cache.bf16_table, cache.codebooks, t,
                                     cache.pos, cache.seq_len, cache.q_end, return_scores=True,
                                     heads=heads)
        pairs = [(0, h) for h in heads]
        check(out, lse, ro, rl, f"t={t}", pairs=pairs)
        s = sc.cpu().numpy()
        l = lse.cpu().numpy()
        for h in heads:
            m_gpu = float(np.exp(s[0, h, lo:lo + 16].astype(np.float64) - l[0, h]).sum())
            m_ref = orc.needle_mass(rs[(0, h)], rl[0, h], lo, lo + 16)
            print(f"  needle mass h={h}: gpu {m_gpu:.6f} oracle {m_ref:.6f}", flush=True)
            assert m_ref > 0.5          # the needle dominates (uniform mass would be 2.4e-4)
            assert abs(m_gpu - m_ref) <= 2e-3
            np.testing.assert_allclose(s[0, h], rs[(0, h)], atol=2e-3, rtol=1e-4)


def test_mixed_serving_batch_sampled():
    """Mixed batch: 64 sequences with lengths U[1024, 16384], T=8, Tc=4, G=32, plus the
    prelude layer coded per step (T=1, Tc=1, G=32); sampled (b, h) pairs."""
    print("\ncase mixed batch B=64", flush=True)
    rl_ = np.random.default_rng(synth.seed_for(5, synth.STREAM_LENGTHS))
    lengths = synth.uniform_lengths(rl_, 64, 1024, 16384)
    pairs = [(0, 0), (17, 4), (40, 15), (63, 9)]
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
