"""Multi-row attention (prefill chunk over a coded prefix; GQA decode) against the float64
oracle, through the C ABI.

Query i of a chunk is the oracle's decode attention over the prefix plus the chunk's
tokens 0 .. i (appended as bf16 tokens after the prefix), at position prefix + i.
Tolerance as for decode: max-abs <= 2e-3 over every element and max-rel <= 1e-2 over
the elements with |oracle| >= 0.2; lse within 1e-4.
"""
import numpy as np
import pytest
import torch

import synth
from cachebuild import build_cache, build_cache_light
from gpu_helpers import attn_close, to_dev
from oracle import lvq_oracle as orc
import parity_log as plog

pytestmark = pytest.mark.gpu


def _dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda")


def _page_tokens(bp, pg, n):
    """Tokens 0..n-1 of bf16 page pg as K, V [T][n][H][d]."""
    return (np.ascontiguousarray(bp[pg][:, :, 0, :n].transpose(0, 2, 1, 3)),
            np.ascontiguousarray(bp[pg][:, :, 1, :n].transpose(0, 2, 1, 3)))


def extended_bf16(cache, ck, cv):
    """The oracle's bf16 pages for prefix + chunk: page 0 and the recent tokens of the
    prefix (read from the prefix's pages) followed by the chunk's tokens ck/cv [b][T][NQ][H][d]."""
    fk, fv, rk, rv, lens = [], [], [], [], []
    NQ = ck[0].shape[1]
    for b in range(cache.B):
        L, qe = int(cache.seq_len[b]), int(cache.q_end[b])
        k0, v0 = _page_tokens(cache.bf16_pages, cache.bf16_table[b, 0], min(8, L))
        base = (qe // 8) * 8
        ks, vs = [], []
        for p0 in range(base, L, 8):
            pg = cache.bf16_table[b, 1 + (p0 - base) // 8]
            k_, v_ = _page_tokens(cache.bf16_pages, pg, min(8, L - p0))
            ks.append(k_)
            vs.append(v_)
        ks.append(ck[b])
        vs.append(cv[b])
        rec_k, rec_v = np.concatenate(ks, axis=1), np.concatenate(vs, axis=1)
        if base == 0:   # the chunk can reach into page 0 only when the prefix is shorter than 8
            n0 = min(8, L + NQ)
            k0, v0 = rec_k[:, :n0], rec_v[:, :n0]
        fk.append(k0)
        fv.append(v0)
        rk.append(rec_k)
        rv.append(rec_v)
        lens.append(L + NQ)
    return synth.pack_bf16_pages_parts(fk, fv, rk, rv, cache.q_end, lens, cache.T, cache.H, cache.d)


def oracle_rows(cache, q_rows, t, ck=None, cv=None, queries=None, pairs=None):
    """out [B][NQ][Hq][d], lse [B][NQ][Hq] (NaN where not computed)."""
    B, NQ = q_rows.shape[0], q_rows.shape[1]
    shp = cache.shape()
    L = cache.seq_len.astype(np.int64)
    if ck is not None:
        bp, lay = extended_bf16(cache, ck, cv)
        bt = lay.bf16_table
    else:
        bp, bt = cache.bf16_pages, cache.bf16_table
    out = np.full((B, NQ, cache.Hq, cache.d), np.nan)
    lse = np.full((B, NQ, cache.Hq), np.nan)
    for i in (range(NQ) if queries is None else queries):
        extra = i + 1 if ck is not None else 0
        o, ls = orc.decode_attn(shp, q_rows[:, i], cache.page_table, cache.index_pages, bp, bt,
                                cache.codebooks, t, L + i if ck is not None else cache.pos,
                                L + extra, cache.q_end, pairs=pairs)
        out[:, i], lse[:, i] = o, ls
    return out, lse


def gpu_rows(dc, cache, q_rows, t, ck=None, cv=None, n_splits=0):
    import sub_bit_loop_amd as lvq
    B, NQ = q_rows.shape[0], q_rows.shape[1]
    shp = lvq.make_rows_shape(B, NQ, cache.H, cache.Hq, cache.d, cache.T, cache.Tc, cache.G, cache.n_sink,
                              dc.page_table.shape[1], dc.bf16_table.shape[1], dc.index_pages.shape[0],
                              dc.bf16_pages.shape[0], int(cache.seq_len.max()), dc.rope_max_len, n_splits)
    pos = cache.seq_len if ck is not None else cache.pos
    kn = vn = None
    if ck is not None:
        kn = _dev(np.stack([k[t] for k in ck]))          # [B][NQ][H][d]
        vn = _dev(np.stack([v[t] for v in cv]))
    out, lse = lvq.lvq_rows_attn(_dev(q_rows), dc.page_table, dc.index_pages, dc.bf16_pages, dc.bf16_table,
                                 dc.codebooks, t, _dev(pos.astype(np.int32)), dc.seq_len, dc.q_end, dc.rope, shp,
                                 k_new=kn, v_new=vn)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def compare(got, ref, label):
    (o, l), (ro, rl) = got, ref
    sel = ~np.isnan(rl)
    ok, mabs, mrel = attn_close(o[sel], ro[sel])
    lerr = float(np.abs(l[sel] - rl[sel]).max())
    plog.line(f"{label}: {int(sel.sum())} rows, max-abs {mabs:.3e} max-rel {mrel:.3e} (|ref| >= 0.2), "
              f"lse max-abs {lerr:.3e}")
    assert ok, f"{label}: output outside tolerance (max-abs {mabs:.3e})"
    assert lerr <= 1e-4, f"{label}: lse error {lerr:.3e}"


def _chunk(seed, B, T, NQ, H, d, Hq):
    rng = np.random.default_rng(seed)
    sc = synth.channel_scales(rng, H, d)
    ck = [synth.f32_to_bf16_bits(synth.gen_kv(rng, T, NQ, H, d, sc)) for _ in range(B)]
    cv = [synth.f32_to_bf16_bits(synth.gen_kv(rng, T, NQ, H, d, sc)) for _ in range(B)]
    q = synth.gen_queries(rng, NQ, B, Hq, d).transpose(1, 0, 2, 3)      # [B][NQ][Hq][d]
    return ck, cv, np.ascontiguousarray(q)


@pytest.mark.parametrize("cfg,lengths,NQ,H,Hq,T,Tc,G,ns,nr,steps", [
    (41, [100, 300], 20, 2, 4, 4, 4, 32, 4, 16, (0, 3)),     # GQA x2, c = 8, ragged row blocks
    (42, [520], 37, 2, 2, 4, 2, 32, 4, 64, (1,)),            # c = 16, three row blocks
    (43, [5, 61], 18, 1, 1, 1, 1, 32, 4, 16, (0,)),          # c = 32; a prefix shorter than a page
])
def test_prefill_chunk_matches_oracle(cfg, lengths, NQ, H, Hq, T, Tc, G, ns, nr, steps):
    plog.case(f"multi-row attention: prefill chunk cfg={cfg} L={lengths} NQ={NQ} H={H} Hq={Hq} T={T} Tc={Tc} G={G}")
    cache = build_cache(cfg, len(lengths), lengths, H, 128, T, Tc, G, ns, nr, Hq=Hq, books="random")
    dc = to_dev(cache, max_seq_len=int(max(lengths)) + NQ)
    ck, cv, q = _chunk(cfg, len(lengths), T, NQ, H, 128, Hq)
    for t in steps:
        compare(gpu_rows(dc, cache, q, t, ck, cv), oracle_rows(cache, q, t, ck, cv), f"t={t}")


@pytest.mark.parametrize("cfg,lengths,H,Hq,T,Tc,G", [
    (44, [64, 333, 1000], 2, 8, 4, 4, 32),                   # 4 query heads per KV head
    (45, [17, 700], 1, 16, 1, 1, 32),                        # 16 heads on one KV head, c = 32
])
def test_gqa_decode_matches_oracle(cfg, lengths, H, Hq, T, Tc, G):
    plog.case(f"multi-row attention: GQA decode cfg={cfg} L={lengths} H={H} Hq={Hq}")
    cache = build_cache(cfg, len(lengths), lengths, H, 128, T, Tc, G, 4, 64, Hq=Hq, books="random")
    dc = to_dev(cache)
    q = np.ascontiguousarray(cache.q[T - 1][:, None])                    # [B][1][Hq][d]
    compare(gpu_rows(dc, cache, q, T - 1), oracle_rows(cache, q, T - 1), f"t={T - 1}")


def test_rows_split_count_does_not_change_the_result():
    """Explicit split counts (one workgroup of chunks, and many) agree with the oracle."""
    cache = build_cache(46, 1, [900], 2, 128, 4, 4, 32, 4, 16, Hq=4, books="random")
    dc = to_dev(cache, max_seq_len=900 + 9)
    ck, cv, q = _chunk(46, 1, 4, 9, 2, 128, 4)
    ref = oracle_rows(cache, q, 2, ck, cv)
    for n in (8, 56):
        compare(gpu_rows(dc, cache, q, 2, ck, cv, n_splits=n), ref, f"splits={n}")


def test_long_chunk_over_short_prefixes_sampled():
    """A chunk much longer than its prefixes: 700 new tokens over prefixes of 100 and 37
    tokens (GQA x2, two row blocks per query position band), so most keys a row sees are
    the chunk's own, causal over many tiles; sampled query positions at the tile and
    row-block edges and the last one, every head."""
    plog.case("multi-row attention: prefill chunk 700 over prefixes [100, 37]")
    NQ = 700
    cache = build_cache(49, 2, [100, 37], 1, 128, 4, 4, 32, 4, 16, Hq=2, books="random")
    dc = to_dev(cache, max_seq_len=100 + NQ)
    ck, cv, q = _chunk(49, 2, 4, NQ, 1, 128, 2)
    got = gpu_rows(dc, cache, q, 3, ck, cv)
    ref = oracle_rows(cache, q, 3, ck, cv, queries=(0, 1, 7, 8, 15, 16, 63, 64, 255, 256, 511, 512, 698, 699))
    compare(got, ref, "t=3")


def test_prefill_chunk_at_32k_sampled():
    """512 new tokens over a 32768-token coded prefix (Ouro-shaped head, 16 heads, MHA), the
    launch the bench times; the oracle checks eight query positions of four heads."""
    plog.case("multi-row attention: prefill chunk 512 over 32K")
    NQ = 512
    cache = build_cache_light(47, 1, [32768], 16, 128, 4, 4, 32, 4, 64)
    dc = to_dev(cache, max_seq_len=32768 + NQ)
    ck, cv, q = _chunk(47, 1, 4, NQ, 16, 128, 16)
    got = gpu_rows(dc, cache, q, 1, ck, cv)
    ref = oracle_rows(cache, q, 1, ck, cv, queries=(0, 1, 15, 16, 255, 256, 500, 511),
                      pairs=[(0, 0), (0, 3), (0, 12), (0, 15)])
    compare(got, ref, "t=1")


def test_gqa_decode_at_32k_sampled():
    """GQA decode at 32K: 8 sequences, 4 KV heads x 4 query heads; every query head of
    sequences 0, 3 and 7."""
    plog.case("multi-row attention: GQA decode B=8 L=32K H=4 Hq=16")
    cache = build_cache_light(48, 8, [32768] * 8, 4, 128, 4, 4, 32, 4, 64, Hq=16)
    dc = to_dev(cache)
    q = np.ascontiguousarray(cache.q[2][:, None])
    got = gpu_rows(dc, cache, q, 2)
    ref = oracle_rows(cache, q, 2, pairs=[(b, h) for b in (0, 3, 7) for h in range(16)])
    compare(got, ref, "t=2")


def test_rows_rejects_bad_arguments():
    import sub_bit_loop_amd as lvq
    cache = build_cache(49, 1, [40], 1, 128, 4, 4, 32, 4, 16, books="random")
    dc = to_dev(cache)
    q = np.zeros((1, 1, 1, 128), np.uint16)
    shp = lvq.make_rows_shape(1, 1, 1, 1, 128, 4, 4, 32, 4, dc.page_table.shape[1], dc.bf16_table.shape[1],
                              dc.index_pages.shape[0], dc.bf16_pages.shape[0], 40, 40)   # rope too short
    with pytest.raises(lvq.LvqError):
        lvq.lvq_rows_attn(_dev(q), dc.page_table, dc.index_pages, dc.bf16_pages, dc.bf16_table, dc.codebooks, 0,
                          dc.pos, dc.seq_len, dc.q_end, dc.rope, shp)
    shp.rope_max_len = dc.rope_max_len
    shp.d = 64
    with pytest.raises((lvq.LvqError, ValueError)):
        lvq.lvq_rows_attn(_dev(q), dc.page_table, dc.index_pages, dc.bf16_pages, dc.bf16_table, dc.codebooks, 0,
                          dc.pos, dc.seq_len, dc.q_end, dc.rope, shp)


def test_decode_attn_routes_wide_groups_to_the_rows_kernel():
    """lvq_decode_attn with 16 query heads per KV head (d = 128) runs on the multi-row
    kernel; the result is the oracle's and the workspace query covers it."""
    from gpu_helpers import gpu_attn
    plog.case("multi-row attention: decode attn, 16 query heads per KV head")
    cache = build_cache(50, 2, [77, 640], 1, 128, 4, 2, 32, 4, 64, Hq=16, books="random")
    dc = to_dev(cache)
    out, lse = gpu_attn(dc, 3)
    ro, rl = cache.oracle_attn(3)
    ok, mabs, mrel = attn_close(out.cpu().numpy(), ro)
    assert ok, f"max-abs {mabs:.3e}"
    assert float(np.abs(lse.cpu().numpy() - rl).max()) <= 1e-4


def test_prefill_chunk_with_an_empty_prefix_and_single_queries():
    """prefix_len = 0 (the chunk attends only to itself) next to a one-token chunk."""
    plog.case("multi-row attention: prefill chunk, empty prefix / one token")
    for cfg, lengths, NQ in ((51, [0, 45], 23), (52, [33], 1)):
        cache = build_cache(cfg, len(lengths), [max(L, 1) for L in lengths], 2, 128, 4, 4, 32, 4, 16, Hq=2,
                            books="random")
        # an empty prefix: zero the sequence's length and coded run (its pages are simply unused)
        cache.seq_len = np.array(lengths, np.int32)
        cache.q_end = np.array([orc.prefill_boundary(L, 16) for L in lengths], np.int32)
        dc = to_dev(cache, max_seq_len=max(lengths) + NQ)
        ck, cv, q = _chunk(cfg, len(lengths), 4, NQ, 2, 128, 2)
        compare(gpu_rows(dc, cache, q, 0, ck, cv), oracle_rows(cache, q, 0, ck, cv), f"cfg={cfg}")


def test_split_products_keep_float32_precision_on_a_sharp_softmax():
    """Queries scaled by 8 (exact in bf16) make every score 8 times larger and the softmax
    sharp.  One float16 product per score (relative error 2^-11 per product) would move
    lse by 1e-2 or more here; the multi-row kernel's hi/lo split products (about 2^-21)
    keep it within the decode tolerance of the oracle, on lvq_decode_attn's multi-row
    route (16 query heads per KV head).  The difference to the per-head kernel's float32
    arithmetic on the same call is recorded."""
    from gpu_helpers import gpu_attn
    plog.case("multi-row attention: queries x8 (sharp softmax), 16 query heads per KV head, split products")
    cache = build_cache(83, 2, [700, 230], 1, 128, 4, 4, 32, 4, 16, Hq=16, books="random")
    bits = cache.q.view(np.uint16).astype(np.uint32) << 16
    cache.q = ((bits.view(np.float32) * np.float32(8.0)).view(np.uint32) >> 16).astype(np.uint16)
    dc = to_dev(cache)
    for t in (0, 3):
        out, lse = gpu_attn(dc, t)
        ro, rl = cache.oracle_attn(t)
        o = out.cpu().numpy()
        ok, mabs, mrel = attn_close(o, ro)
        lerr = float(np.abs(lse.cpu().numpy() - rl).max())
        o2, l2, _ = gpu_attn(dc, t, scores=True)
        dph = float(np.abs(o - o2.cpu().numpy()).max())
        plog.line(f"t={t}: max-abs {mabs:.3e} max-rel {mrel:.3e} (|ref| >= 0.2), lse max-abs {lerr:.3e}; "
                  f"multi-row vs per-head kernel max-abs {dph:.3e}")
        assert ok, f"t={t}: output outside tolerance (max-abs {mabs:.3e})"
        assert lerr <= 1e-4, f"t={t}: lse error {lerr:.3e}"


def test_multirow_decode_over_many_ragged_sequences():
    """70 sequences with lengths U[1, 400], one KV head with 16 query heads (the multi-row
    route of lvq_decode_attn): automatic, one-workgroup and 4000-wave splits all match the
    oracle and agree closely with each other; the same split twice gives identical bits.
    Short sequences are mostly bf16 sink and recent tiles, which the split weighs as four
    coded tiles each, so ranges end inside them; the 4000-wave split gives most waves an
    empty range and sequences many records (the deep merge)."""
    from gpu_helpers import gpu_attn
    plog.case("multi-row decode, B=70 lengths U[1,400], H=1 Hq=16, splits 0/8/4000")
    rl_ = np.random.default_rng(synth.seed_for(84, synth.STREAM_LENGTHS))
    lengths = synth.uniform_lengths(rl_, 70, 1, 400)
    cache = build_cache(84, 70, lengths, 1, 128, 4, 4, 32, 4, 16, Hq=16, books="random", index="random")
    dc = to_dev(cache)
    t = 1
    ro, rl = cache.oracle_attn(t)
    outs = []
    for S in (0, 8, 4000):
        out, lse = gpu_attn(dc, t, n_splits=S)
        o = out.cpu().numpy()
        ok, mabs, mrel = attn_close(o, ro)
        lerr = float(np.abs(lse.cpu().numpy() - rl).max())
        plog.line(f"splits={S}: max-abs {mabs:.3e} max-rel {mrel:.3e} (|ref| >= 0.2), lse max-abs {lerr:.3e}")
        assert ok, f"splits={S}: output outside tolerance (max-abs {mabs:.3e})"
        assert lerr <= 1e-4, f"splits={S}: lse error {lerr:.3e}"
        outs.append(o)
    for o in outs[1:]:
        np.testing.assert_allclose(o, outs[0], rtol=2e-5, atol=2e-6)
    again, _ = gpu_attn(dc, t, n_splits=4000)
    np.testing.assert_array_equal(again.cpu().numpy(), outs[2])
