"""GPU parity of grouped-query decode (2, 4 and 8 query heads per KV head, d = 128):
lvq_decode_attn routes 2 and 4 heads per KV head to the kernel that shares each key's
dequantisation and rotation over the KV head's query heads, and 8 to the multi-row
kernel (the heads as the rows of its matrix-core products).  Same tolerance as the per-head decode
tests: max-abs <= 2e-3 over every output element, max-rel <= 1e-2 where |oracle| >= 0.2,
lse within 1e-4.
lvq_decode_scores keeps the per-head kernel on the same shapes, so the two kernels are
also compared with each other."""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from cachebuild import build_cache, build_cache_light
from gpu_helpers import attn_close, gpu_attn, to_dev
from oracle import lvq_oracle as orc
import parity_log as plog
from test_gpu_attn import check

pytestmark = pytest.mark.gpu


GROUPED = [  # config, lengths, H, query heads per KV head, T, Tc, G, n_sink, n_recent
    (60, [37, 300, 1000], 2, 4, 4, 4, 32, 4, 16),      # c = 8, ragged lengths
    (61, [515, 260], 1, 4, 4, 2, 32, 0, 16),           # c = 16, no sink
    (62, [1000, 33], 2, 4, 1, 1, 32, 4, 64),           # prelude layer: Tc = 1, c = 32
    (63, [1, 8, 19], 1, 4, 4, 4, 32, 4, 64),           # shorter than sink + recent: all bf16
    (64, [0, 45, 0], 2, 4, 4, 4, 32, 4, 16),           # empty batch slots: out 0, lse -inf
    (65, [300, 129], 2, 4, 8, 4, 32, 8, 64),           # two loop blocks, n_sink = 8
    (69, [37, 300, 1000], 2, 2, 4, 4, 32, 4, 16),      # 2 heads per KV head, c = 8
    (70, [515, 0, 260], 3, 2, 4, 2, 32, 0, 64),        # 2 heads per KV head, c = 16, an empty slot
    (71, [1000, 8], 1, 2, 1, 1, 32, 8, 16),            # 2 heads per KV head, c = 32
    (80, [37, 300, 1000], 1, 8, 4, 4, 32, 4, 16),      # 8 heads per KV head (multi-row route), c = 8
    (81, [515, 0, 260], 2, 8, 4, 2, 32, 0, 64),        # 8 heads per KV head (multi-row route), c = 16
    (82, [1000, 8], 1, 8, 1, 1, 32, 8, 16),            # 8 heads per KV head (multi-row route), c = 32
]


@pytest.mark.parametrize("cfg,lengths,H,g,T,Tc,G,ns,nr", GROUPED)
def test_grouped_decode_matches_oracle(cfg, lengths, H, g, T, Tc, G, ns, nr):
    plog.case(f"grouped decode ({g} query heads per KV head) cfg={cfg} L={lengths} H={H} Hq={g * H} "
              f"T={T} Tc={Tc} G={G} n_sink={ns} n_recent={nr}; every step, every (b, head)")
    cache = build_cache(cfg, len(lengths), lengths, H, 128, T, Tc, G, ns, nr, Hq=g * H, books="random")
    dc = to_dev(cache)
    for t in range(T):
        out, lse = gpu_attn(dc, t)
        ro, rl = cache.oracle_attn(t)
        check(out, lse, ro, rl, f"t={t}")
        # the per-head kernel (lvq_decode_scores) on the same call
        o2, l2, _ = gpu_attn(dc, t, scores=True)
        ok, mabs, _ = attn_close(out.cpu().numpy(), o2.cpu().numpy(), atol=2e-5, rtol=1e-4)
        assert ok, f"t={t}: grouped and per-head kernels differ by {mabs:.3e}"


def test_grouped_split_counts():
    """70 sequences with lengths U[1, 400], 2 KV heads x 4 query heads: automatic, one
    workgroup and 4000-wave splits (most quads then take empty ranges) all match the oracle
    and agree closely with each other; the same split twice gives identical bits."""
    plog.case("grouped decode, B=70 lengths U[1,400], H=2 Hq=8, splits 0/16/4000")
    rl_ = np.random.default_rng(synth.seed_for(66, synth.STREAM_LENGTHS))
    lengths = synth.uniform_lengths(rl_, 70, 1, 400)
    cache = build_cache(66, 70, lengths, 2, 128, 4, 4, 32, 4, 16, Hq=8, books="random", index="random")
    dc = to_dev(cache)
    t = 2
    ro, rl = cache.oracle_attn(t)
    outs = []
    for S in (0, 16, 4000):
        out, lse = gpu_attn(dc, t, n_splits=S)
        check(out, lse, ro, rl, f"splits={S}")
        outs.append(out.cpu().numpy())
    for o in outs[1:]:
        np.testing.assert_allclose(o, outs[0], rtol=2e-5, atol=2e-6)
    again, _ = gpu_attn(dc, t, n_splits=4000)
    np.testing.assert_array_equal(again.cpu().numpy(), outs[2])


def test_grouped_index_pool_beyond_4gib():
    """The grouped kernel's 64-bit page addressing: the same pages at the top of a pool over
    4 GiB give the same bits as the compact pool."""
    plog.case("grouped decode, index pool over 4 GiB: bit-identical to the compact pool")
    cache = build_cache(67, 1, [2000], 2, 128, 4, 4, 32, 4, 64, Hq=8, books="random", index="random")
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


@pytest.mark.parametrize("H,Hq", [(4, 16), (8, 16), (2, 16)])
def test_grouped_decode_at_32k(H, Hq):
    """The benchmark's grouped shapes: B=8 sequences of 32768 tokens, 16 query heads over 8,
    4 or 2 KV heads (grouped, grouped and multi-row routes), d=128, T=4, Tc=4, G=32, 4 sink
    + 64 recent, shuffled pages, automatic split.  The oracle checks every query head of sequences 0, 3 and 7 at two loop steps;
    all 128 (b, head) outputs are compared with the per-head kernel."""
    plog.case(f"grouped decode at 32K: B=8 L=32768 H={H} Hq={Hq} d=128 T=4 Tc=4 G=32; "
              "oracle on sequences 0, 3, 7 (all heads), per-head kernel on all pairs")
    cache = build_cache_light(68, 8, [32768] * 8, H, 128, 4, 4, 32, 4, 64, Hq=Hq)
    dc = to_dev(cache)
    pairs = [(b, h) for b in (0, 3, 7) for h in range(16)]
    for t in (0, 3):
        out, lse = gpu_attn(dc, t)
        ro, rl = orc.decode_attn(cache.shape(), cache.q[t], cache.page_table, cache.index_pages,
                                 cache.bf16_pages, cache.bf16_table, cache.codebooks, t, cache.pos,
                                 cache.seq_len, cache.q_end, pairs=pairs)
        check(out, lse, ro, rl, f"t={t}", pairs=pairs)
        o2, l2, _ = gpu_attn(dc, t, scores=True)
        ok, mabs, _ = attn_close(out.cpu().numpy(), o2.cpu().numpy(), atol=2e-5, rtol=1e-4)
        plog.line(f"t={t}: grouped vs per-head kernel over all 128 (b, head) rows: max-abs {mabs:.3e}")
        assert ok, f"t={t}: grouped and per-head kernels differ by {mabs:.3e}"
        lerr = float(np.abs(lse.cpu().numpy() - l2.cpu().numpy()).max())
        assert lerr <= 1e-4
