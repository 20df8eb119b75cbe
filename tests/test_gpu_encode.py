"""GPU encoder parity against the float64 oracle, through the C ABI.

Indices must be bit-exact, except where the oracle's own near-tie set N(x)
(distance within 1e-5 relative of the best) has more than one member and the
GPU picked another member of it; every such vector is printed.
"""
import numpy as np
import pytest
import torch

import synth
from cachebuild import build_cache
from oracle import lvq_oracle as orc
import parity_log as plog

pytestmark = pytest.mark.gpu


def dev(x):
    a = np.ascontiguousarray(x)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def gpu_encode(kv_bits, cb_bits, kv_sel, T, Tc, G):
    import sub_bit_loop_amd as lvq
    out = lvq.lvq_encode(dev(kv_bits), dev(cb_bits), kv_sel, T, Tc, G)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def near_tie_ok(got, ref_idx, n_near, D_of, d2=None):
    """Mismatches allowed only inside the oracle near-tie set N(x); every one is listed in
    the parity record as (beta, n, h, g, i*, i_gpu, D1, D2).  Returns their count."""
    mism = np.argwhere(got != ref_idx)
    listed = 0
    for pos in mism:
        pos = tuple(int(x) for x in pos)
        assert n_near[pos] > 1, f"mismatch outside the near-tie band at {pos}: gpu {got[pos]} oracle {ref_idx[pos]}"
        d_gpu, d1 = D_of(pos, int(got[pos]))
        assert d_gpu - d1 <= 1e-5 * d1, f"gpu index {got[pos]} outside N(x) at {pos}"
        beta, n, h, g = pos
        d2s = f" D2={float(d2[pos]):.9g}" if d2 is not None else ""
        plog.line(f"near tie (beta={beta}, n={n}, h={h}, g={g}): i*={int(ref_idx[pos])} i_gpu={int(got[pos])} "
                  f"D1={d1:.9g}{d2s} D(i_gpu)={d_gpu:.9g}")
        listed += 1
    return listed


CASES = [  # T, Tc, G, d, N, H
    (4, 2, 16, 64, 512, 1),     # the tiny configuration (c = 8)
    (4, 4, 32, 128, 203, 2),    # c = 8, ragged token tail
    (4, 2, 32, 128, 96, 1),     # c = 16
    (1, 1, 32, 128, 150, 2),    # prelude layer coded per step, c = 32
    (8, 4, 32, 128, 40, 1),     # deeper loop, two blocks
    (4, 4, 16, 64, 72, 1),      # c = 4
    (4, 1, 16, 64, 33, 1),      # c = 16, G = 16
    (2, 2, 32, 64, 17, 2),      # d = 64, c = 16
    (4, 4, 32, 128, 1, 3),      # a single token, an odd head count
    (4, 2, 16, 128, 65, 5),     # five heads (no power of two), one token past two tiles
    (1, 1, 32, 64, 70, 3),      # d = 64, c = 32: two groups, so two-wave workgroups
]


@pytest.mark.parametrize("T,Tc,G,d,N,H", CASES)
def test_encode_matches_oracle(T, Tc, G, d, N, H):
    plog.case(f"encode T={T} Tc={Tc} G={G} d={d} N={N} H={H}, k-means books on 4096 samples, "
              f"every vector of K and V")
    cache = build_cache(21, 1, [N], H, d, T, Tc, G, 4, 16, book_samples=4096, index="random")
    for kv_sel, toks in ((0, cache.k_tokens[0]), (1, cache.v_tokens[0])):
        got = gpu_encode(toks, cache.codebooks, kv_sel, T, Tc, G)
        ref = orc.encode(toks, cache.codebooks, kv_sel, T, Tc, G)
        J = orc.joint_vectors(orc.bf16_to_f64(toks), Tc, G)
        C = orc.joint_codewords(orc.bf16_to_f64(cache.codebooks)[:, kv_sel])

        def D_of(pos, k):
            beta, n, h, g = pos
            return float(((J[beta, n, h, g] - C[beta, h, g, k]) ** 2).sum()), float(ref.d1[pos])

        n_tie = near_tie_ok(got, ref.idx, ref.n_near, D_of, ref.d2)
        plog.line(f"{'KV'[kv_sel]}: {got.size} vectors, {int((got == ref.idx).sum())} bit-exact, "
                  f"{n_tie} listed near ties, {int((ref.n_near > 1).sum())} oracle near-tie sets")


def test_encode_duplicate_identity_and_product_books():
    """Exact ties (duplicated codewords) must return the lowest index; codewords equal
    to data vectors must be found exactly (distance 0); product books separate."""
    T, Tc, G, d, N, H = 4, 2, 16, 64, 128, 1
    c = G // Tc
    nblk, ng = T // Tc, d // c
    rng = np.random.default_rng(5)
    kv = synth.f32_to_bf16_bits(rng.standard_normal((T, N, H, d)).astype(np.float32))
    X = orc.bf16_to_f64(kv)
    J = orc.joint_vectors(X, Tc, G)                          # [nblk][N][H][ng][G]
    # identity: codeword k = joint vector of token k (k < N), the rest far away
    cbf = 40.0 + rng.standard_normal((nblk, 2, H, ng, Tc, 256, c))
    for beta in range(nblk):
        for g in range(ng):
            for tau in range(Tc):
                cbf[beta, :, 0, g, tau, :N] = J[beta, :, 0, g, tau * c:(tau + 1) * c][None]
    # duplicates: codeword 200 and 250 copy codeword 3; 201 copies 7
    cbf[..., 200, :] = cbf[..., 3, :]
    cbf[..., 250, :] = cbf[..., 3, :]
    cbf[..., 201, :] = cbf[..., 7, :]
    cb = synth.f32_to_bf16_bits(cbf.astype(np.float32))
    got = gpu_encode(kv, cb, 0, T, Tc, G)
    np.testing.assert_array_equal(got, np.broadcast_to(np.arange(N)[None, :, None, None], got.shape))
    # a query sitting exactly on a duplicated codeword: lowest index
    kv2 = kv.copy()
    ref = orc.encode(kv2, cb, 1, T, Tc, G)
    got2 = gpu_encode(kv2, cb, 1, T, Tc, G)
    np.testing.assert_array_equal(got2, ref.idx)
    # product books (Tc = 2): codeword 16a + b = (A_a, B_b)
    A = rng.standard_normal((nblk, 2, H, ng, 16, c))
    Bq = rng.standard_normal((nblk, 2, H, ng, 16, c))
    pb = np.zeros((nblk, 2, H, ng, Tc, 256, c))
    for a_ in range(16):
        for b_ in range(16):
            pb[..., 0, 16 * a_ + b_, :] = A[..., a_, :]
            pb[..., 1, 16 * a_ + b_, :] = Bq[..., b_, :]
    pbb = synth.f32_to_bf16_bits(pb.astype(np.float32))
    ref = orc.encode(kv, pbb, 0, T, Tc, G)
    got = gpu_encode(kv, pbb, 0, T, Tc, G)
    ok = ref.n_near == 1
    np.testing.assert_array_equal(got[ok], ref.idx[ok])


def test_encode_zero_vectors_and_zero_codeword():
    """x = 0 makes every expanded distance |C|^2 >= 0 (the float32 fast path cannot
    decide); the float64 path must still return the lowest-norm codeword."""
    T, Tc, G, d, N, H = 4, 4, 32, 128, 48, 1
    rng = np.random.default_rng(6)
    kv = np.zeros((T, N, H, d), dtype=np.uint16)
    cb = synth.random_codebooks(rng, T, Tc, G, H, d)
    ref = orc.encode(kv, cb, 0, T, Tc, G)
    got = gpu_encode(kv, cb, 0, T, Tc, G)
    np.testing.assert_array_equal(got, ref.idx)


@pytest.mark.parametrize("e", [-70, -60, 60, 64])
@pytest.mark.parametrize("Tc,G,d", [(2, 16, 64), (4, 32, 128)])
def test_encode_extreme_magnitudes(e, Tc, G, d):
    """Keys, values and codewords all scaled by 2^e (exact in bf16).  At 2^-70 the products
    fall below the float32 normal range (they may be flushed), at 2^-60 some of them do,
    at 2^60 some squared norms and at 2^64 all of them overflow float32.  The indices must
    still be the float64 nearest codeword: the float32 decision is trusted only where its
    error bound holds, and the float64 pass decides the rest."""
    T, N, H = 4, 96, 1
    plog.case(f"encode extreme magnitudes x 2^{e}: T={T} Tc={Tc} G={G} d={d} N={N} H={H}")
    rng = np.random.default_rng(synth.seed_for(9, synth.STREAM_K))
    sc = synth.channel_scales(rng, H, d)
    kv = synth.gen_kv(rng, T, N, H, d, sc)
    samp = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(synth.gen_kv(rng, T, 1024, H, d, sc)))
    books = synth.codebooks_from_samples(samp, Tc, G, 91)                  # bf16 bits [nblk][H][ng][Tc][256][c]
    scale = np.float32(2.0 ** e)
    kv_s = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(kv)) * scale)
    cb_s = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(np.stack([books, books], axis=1)) * scale)
    assert np.isfinite(synth.bf16_bits_to_f32(kv_s)).all() and np.isfinite(synth.bf16_bits_to_f32(cb_s)).all()
    got = gpu_encode(kv_s, cb_s, 0, T, Tc, G)
    ref = orc.encode(kv_s, cb_s, 0, T, Tc, G)
    n_exact = int((got == ref.idx).sum())
    plog.line(f"{got.size} vectors, {n_exact} bit-exact")
    np.testing.assert_array_equal(got, ref.idx)


@pytest.mark.parametrize("Tc,G", [(4, 32), (2, 16)])
def test_encode_full_size_slab(Tc, G):
    """Prefill-encode shape: T=4 steps x 32768 tokens x 16 heads x d=128, the whole tensor
    encoded on the GPU; every vector of one whole (block, head) slab (32768 tokens x 16
    groups = 524288 vectors) checked against the oracle, plus 4096 vectors sampled over
    the rest.  The slab holds vectors whose two best codewords lie within the near-tie
    band (D2 - D1 <= 1e-5 D1, below the float32 error bound of the expanded distances, so
    the kernel can only certify them by its float64 recomputation); every one of them
    must still be exact."""
    T, N, H, d = 4, 32768, 16, 128
    plog.case(f"encode full size T=4 N=32768 H=16 d=128 Tc={Tc} G={G}: one whole (block, head) slab "
              f"+ 4096 sampled vectors")
    rng = np.random.default_rng(synth.seed_for(4, synth.STREAM_K))
    sc = synth.channel_scales(rng, H, d)
    kv = synth.f32_to_bf16_bits(synth.gen_kv(rng, T, N, H, d, sc))
    rb = np.random.default_rng(synth.seed_for(4, synth.STREAM_BOOKS))
    samp = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(synth.gen_kv(rb, T, 4096, H, d, sc)))
    bk = synth.codebooks_from_samples(samp, Tc, G, 77, device="cuda", dtype=torch.float32)
    cb = np.ascontiguousarray(np.stack([bk, bk], axis=1))
    got = gpu_encode(kv, cb, 0, T, Tc, G)
    c = G // Tc
    nblk, ng = T // Tc, d // c
    X = orc.bf16_to_f64(kv)
    C = orc.joint_codewords(orc.bf16_to_f64(cb)[:, 0])
    # the whole slab (beta = nblk - 1, h = 5): every token and group
    beta, h = nblk - 1, 5
    J = orc.joint_vectors(X[beta * Tc:(beta + 1) * Tc][:, :, h:h + 1], Tc, G)[0, :, 0]   # [N][ng][G]
    n_tie, n_tight, n_tight_ok, n_exact = 0, 0, 0, 0
    for g in range(ng):
        r = orc.nearest_codeword(J[:, g], C[beta, h, g])
        gg = got[beta, :, h, g].astype(np.int64)
        gap = r.d2 - r.d1
        tight = (gap <= 1e-5 * r.d1) & (gap > 1e-12 * r.d1)
        n_tight += int(tight.sum())
        n_tight_ok += int((gg[tight] == r.idx[tight]).sum())
        n_exact += int((gg == r.idx).sum())
        for n in np.nonzero(gg != r.idx)[0]:
            dk = float(((J[n, g] - C[beta, h, g, gg[n]]) ** 2).sum())
            assert r.n_near[n] > 1 and dk - r.d1[n] <= 1e-5 * r.d1[n], \
                f"mismatch at (beta={beta}, n={n}, h={h}, g={g}): gpu {gg[n]} oracle {r.idx[n]}"
            plog.line(f"near tie (beta={beta}, n={n}, h={h}, g={g}): i*={int(r.idx[n])} i_gpu={int(gg[n])} "
                      f"D1={r.d1[n]:.9g} D2={r.d2[n]:.9g} D(i_gpu)={dk:.9g}")
            n_tie += 1
    plog.line(f"slab (beta={beta}, h={h}): {N * ng} vectors, {n_exact} bit-exact, {n_tie} listed near ties; "
              f"{n_tight} vectors with 1e-12 D1 < D2 - D1 <= 1e-5 D1, {n_tight_ok} of them exact")
    assert n_tight > 0, "the slab should hold vectors inside the near-tie band"
    assert n_tight_ok == n_tight, "a near-tie vector was not resolved exactly (float64 recomputation)"
    # 4096 vectors sampled over the whole tensor
    srng = np.random.default_rng(9)
    picks = np.stack([srng.integers(0, nblk, 4096), srng.integers(0, N, 4096),
                      srng.integers(0, H, 4096), srng.integers(0, ng, 4096)], 1)
    n_bad = 0
    for beta_, n, h_, g in picks:
        x = np.concatenate([X[beta_ * Tc + tau, n, h_, g * c:(g + 1) * c] for tau in range(Tc)])
        r = orc.nearest_codeword(x[None], C[beta_, h_, g])
        k = int(got[beta_, n, h_, g])
        if k != r.idx[0]:
            dk = float(((x - C[beta_, h_, g, k]) ** 2).sum())
            assert r.n_near[0] > 1 and dk - r.d1[0] <= 1e-5 * r.d1[0], \
                f"mismatch at {(beta_, n, h_, g)}: gpu {k} oracle {r.idx[0]}"
            plog.line(f"near tie (beta={beta_}, n={n}, h={h_}, g={g}): i*={int(r.idx[0])} i_gpu={k} "
                      f"D1={r.d1[0]:.9g} D2={r.d2[0]:.9g} D(i_gpu)={dk:.9g}")
            n_bad += 1
    plog.line(f"sample: 4096 vectors, {4096 - n_bad} bit-exact, {n_bad} listed near ties")


def test_encode_pages_and_reencode():
    """lvq_encode_pages scatters rows to the right (page, slot, half); lvq_reencode_pages
    codes whole bf16 pages (all steps, K and V) like the oracle."""
    import sub_bit_loop_amd as lvq
    T, Tc, G, d, H = 8, 4, 32, 128, 2
    cache = build_cache(22, 2, [80, 45], H, d, T, Tc, G, 4, 16, book_samples=1024)
    c = G // Tc
    nblk, ng = T // Tc, d // c
    P = 40
    rng = np.random.default_rng(3)
    # encode_pages: 64 tokens of sequence 0 into 8 scattered pages
    toks = cache.k_tokens[0][:, :64]
    pages = rng.permutation(P)[:8].astype(np.int32)
    ip = torch.zeros((P, nblk, H, 2, 8, ng), dtype=torch.uint8, device="cuda")
    lvq.lvq_encode_pages(dev(toks), dev(cache.codebooks), 0, T, Tc, G, dev(pages), ip)
    torch.cuda.synchronize()
    ref = np.zeros((P, nblk, H, 2, 8, ng), dtype=np.uint8)
    r = orc.encode(toks, cache.codebooks, 0, T, Tc, G)
    assert (r.n_near <= 1).all()
    orc.scatter_index_pages(r.idx, 0, pages, ref)
    np.testing.assert_array_equal(ip.cpu().numpy(), ref)
    # reencode: the recent bf16 pages of both sequences into fresh coded pages
    src, dst, toks_k, toks_v = [], [], [], []
    for b in range(2):
        row = cache.bf16_table[b]
        for j in range(1, len(row)):
            if row[j] < 0:
                continue
            lp = int(cache.q_end[b]) // 8 + j - 1
            if (lp + 1) * 8 > cache.seq_len[b]:
                continue              # only full pages
            src.append(int(row[j]))
            dst.append(len(dst) * 3 + 1)
            toks_k.append(cache.k_tokens[b][:, lp * 8:lp * 8 + 8])
            toks_v.append(cache.v_tokens[b][:, lp * 8:lp * 8 + 8])
    ip2 = torch.zeros((3 * len(dst) + 2, nblk, H, 2, 8, ng), dtype=torch.uint8, device="cuda")
    lvq.lvq_reencode_pages(dev(cache.bf16_pages), dev(np.array(src, np.int32)),
                           dev(np.array(dst, np.int32)), dev(cache.codebooks), T, Tc, G, ip2)
    torch.cuda.synchronize()
    got = ip2.cpu().numpy()
    ref2 = np.zeros_like(got)
    for kv, toks in ((0, toks_k), (1, toks_v)):
        allt = np.concatenate(toks, axis=1)
        r = orc.encode(allt, cache.codebooks, kv, T, Tc, G)
        assert (r.n_near <= 1).all()
        orc.scatter_index_pages(r.idx, kv, np.array(dst, np.int32), ref2)
    np.testing.assert_array_equal(got, ref2)


def test_page_ids_out_of_range_are_skipped():
    """Chunk pages of lvq_encode_pages and source or destination pages of
    lvq_reencode_pages that are negative or past their pool are skipped: nothing is
    written for them, and every other page is coded as the oracle codes it."""
    import sub_bit_loop_amd as lvq
    T, Tc, G, d, H = 4, 4, 32, 128, 2
    cache = build_cache(23, 1, [64], H, d, T, Tc, G, 4, 16, book_samples=1024)
    c = G // Tc
    nblk, ng = T // Tc, d // c
    P = 12
    toks = cache.k_tokens[0][:, :64]
    pages = np.array([3, -1, 7, P, 0, 11, -5, P + 100], dtype=np.int32)
    ip = torch.full((P, nblk, H, 2, 8, ng), 0xA5, dtype=torch.uint8, device="cuda")
    lvq.lvq_encode_pages(dev(toks), dev(cache.codebooks), 1, T, Tc, G, dev(pages), ip)
    torch.cuda.synchronize()
    ref = np.full((P, nblk, H, 2, 8, ng), 0xA5, dtype=np.uint8)
    r = orc.encode(toks, cache.codebooks, 1, T, Tc, G)
    ok = (pages >= 0) & (pages < P)
    for j in np.nonzero(ok)[0]:
        ref[pages[j], :, :, 1] = r.idx[:, 8 * j:8 * j + 8].transpose(0, 2, 1, 3)
    np.testing.assert_array_equal(ip.cpu().numpy(), ref)
    # re-encode: the sink copy of tokens 0..7 into coded pages, with invalid entries mixed in
    nbf = cache.bf16_pages.shape[0]
    sp = int(cache.bf16_table[0, 0])
    src = np.array([sp, -1, sp, nbf, sp], dtype=np.int32)
    dst = np.array([2, 5, -1, 6, P], dtype=np.int32)
    ip2 = torch.full((P, nblk, H, 2, 8, ng), 0x5A, dtype=torch.uint8, device="cuda")
    lvq.lvq_reencode_pages(dev(cache.bf16_pages), dev(src), dev(dst), dev(cache.codebooks), T, Tc, G, ip2)
    torch.cuda.synchronize()
    got = ip2.cpu().numpy()
    ref2 = np.full_like(got, 0x5A)
    k0 = cache.k_tokens[0][:, :8]
    v0 = cache.v_tokens[0][:, :8]
    for kv, tk in ((0, k0), (1, v0)):
        rr = orc.encode(tk, cache.codebooks, kv, T, Tc, G)
        ref2[2, :, :, kv] = rr.idx[:, 0:8].transpose(0, 2, 1, 3)
    np.testing.assert_array_equal(got, ref2)


def test_reencode_layers_matches_per_layer_and_oracle():
    """lvq_reencode_pages_layers over 50 layers (two launches of at most 48) writes
    exactly what one lvq_reencode_pages call per layer writes, honours each layer's
    own pool bounds, and matches the oracle."""
    import sub_bit_loop_amd as lvq
    T, Tc, G, d, H = 4, 2, 16, 64, 1
    c = G // Tc
    nblk, ng = T // Tc, d // c
    n_layers = 50
    rng = np.random.default_rng(11)
    src = np.array([3, 0, 5, -1, 2, 1], np.int32)
    dst = np.array([7, 1, 2, 4, 9, 3], np.int32)   # page 9 exists in odd layers only
    layers, host = [], []
    for l in range(n_layers):
        n_bf, n_ix = 6, 9 + (l % 2)
        scales = synth.channel_scales(rng, H, d)
        toks = np.stack([synth.f32_to_bf16_bits(synth.gen_kv(rng, T, 8, H, d, scales)) for _ in range(2 * n_bf)])
        bp = toks.reshape(n_bf, 2, T, 8, H, d).transpose(0, 2, 4, 1, 3, 5).copy()   # [P][T][H][2][8][d]
        cb = synth.random_codebooks(rng, T, Tc, G, H, d)
        ip0 = rng.integers(0, 256, size=(n_ix, nblk, H, 2, 8, ng), dtype=np.uint8)
        layers.append((dev(bp), dev(cb), dev(ip0)))
        host.append((bp, cb, ip0))
    per_layer = [torch.from_numpy(h[2]).cuda() for h in host]
    s_d, d_d = dev(src), dev(dst)
    print(f"\ncase layers={n_layers} T={T} Tc={Tc} G={G} d={d} H={H} pages={len(src)}", flush=True)
    lvq.lvq_reencode_pages_layers(layers, s_d, d_d, T, Tc, G)
    for l in range(n_layers):
        lvq.lvq_reencode_pages(layers[l][0], s_d, d_d, layers[l][1], T, Tc, G, per_layer[l])
    torch.cuda.synchronize()
    for l in range(n_layers):
        np.testing.assert_array_equal(layers[l][2].cpu().numpy(), per_layer[l].cpu().numpy(),
                                      err_msg=f"layer {l}")
    for l in (0, 1, 47, 48, 49):
        bp, cb, ip0 = host[l]
        ref = ip0.copy()
        ok = [(s, t) for s, t in zip(src, dst) if 0 <= s < bp.shape[0] and 0 <= t < ref.shape[0]]
        for kv in (0, 1):
            allt = np.concatenate([bp[s, :, :, kv].transpose(0, 2, 1, 3) for s, _ in ok], axis=1)
            r = orc.encode(allt, cb, kv, T, Tc, G)
            assert (r.n_near <= 1).all()
            orc.scatter_index_pages(r.idx, kv, np.array([t for _, t in ok], np.int32), ref)
        np.testing.assert_array_equal(layers[l][2].cpu().numpy(), ref, err_msg=f"layer {l} vs oracle")


def test_binding_refuses_mismatched_shapes():
    """Tensors whose shape does not match the call's sizes are refused before a launch."""
    import sub_bit_loop_amd as lvq
    T, Tc, G, d, H, N = 4, 4, 32, 128, 2, 16
    kv = torch.zeros((T, N, H, d), dtype=torch.int16, device="cuda")
    good = torch.zeros((1, 2, H, 16, Tc, 256, 8), dtype=torch.int16, device="cuda")
    bad = torch.zeros((1, 2, H, 8, Tc, 256, 8), dtype=torch.int16, device="cuda")     # ng = 8, not 16
    with pytest.raises(ValueError, match="codebooks"):
        lvq.lvq_encode(kv, bad, 0, T, Tc, G)
    with pytest.raises(ValueError, match="idx"):
        lvq.lvq_encode(kv, good, 0, T, Tc, G, idx=torch.empty((1, N, H, 8), dtype=torch.uint8, device="cuda"))
    bp = torch.zeros((3, T, H, 2, 8, d), dtype=torch.int16, device="cuda")
    ip_bad = torch.zeros((3, 1, H, 2, 8, 8), dtype=torch.uint8, device="cuda")
    pages = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError, match="index_pages"):
        lvq.lvq_reencode_pages_layers([(bp, good, ip_bad)], pages, pages, T, Tc, G)
    with pytest.raises(ValueError, match="bf16_pages"):
        lvq.lvq_reencode_pages(bp[:, :2].contiguous(), pages, pages, good, T, Tc, G,
                               torch.zeros((3, 1, H, 2, 8, 16), dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
