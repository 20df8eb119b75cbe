"""GPU codebook builder (k-means++ seeding + Lloyd iterations) against the oracle:
bf16 codebooks bit-exact."""
import numpy as np
import pytest

import synth
from oracle import lvq_oracle as orc

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _samples(seed, T, S, H, d):
    rng = np.random.default_rng(seed)
    sc = synth.channel_scales(rng, H, d)
    return synth.f32_to_bf16_bits(synth.gen_kv(rng, T, S, H, d, sc)), rng


def _gpu_build(bits, draws, kv_sel, T, Tc, G, n_iter, codebooks=None, weights=None):
    import sub_bit_loop_amd as lvq
    dev = torch.device("cuda:0")
    x = torch.from_numpy(bits.view(np.int16)).to(dev)
    u = torch.from_numpy(draws).to(dev)
    cb = None if codebooks is None else torch.from_numpy(codebooks.view(np.int16)).to(dev)
    w = None if weights is None else torch.from_numpy(weights).to(dev)
    out = lvq.lvq_build_codebooks(x, u, kv_sel, T, Tc, G, n_iter, codebooks=cb, weights=w)
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy().view(np.uint16)


def books_desc(nblk, ng):
    return f"(block, head, group) in [0, {nblk}) x [0, 16) x [0, {ng})"


def _compare(gpu_half, ref, books):
    for (beta, h, g) in books:
        got, want = gpu_half[beta, h, g], ref[beta, h, g]
        bad = np.argwhere(got != want)
        assert len(bad) == 0, f"book {(beta, h, g)}: {len(bad)} codeword elements differ, first {bad[:4]}"


@pytest.mark.parametrize("T,Tc,G,S,H,d,n_iter", [
    (4, 2, 16, 600, 2, 64, 4),      # 0.5 bit, two blocks
    (4, 4, 32, 500, 1, 128, 3),     # 0.25 bit
    (1, 1, 32, 300, 1, 64, 2),      # prelude layer coded per step (c = 32)
    (4, 4, 16, 280, 1, 64, 2),      # c = 4
])
def test_builder_matches_oracle(T, Tc, G, S, H, d, n_iter):
    print(f"\ncase build T={T} Tc={Tc} G={G} S={S} H={H} d={d} iters={n_iter}", flush=True)
    bits, rng = _samples(61, T, S, H, d)
    nblk, ng = T // Tc, d // (G // Tc)
    draws = rng.random((nblk, H, ng, 256))
    out = _gpu_build(bits, draws, 0, T, Tc, G, n_iter)
    ref = orc.build_codebooks(bits, draws, Tc, G, n_iter)
    _compare(out[:, 0], ref, [(b, h, g) for b in range(nblk) for h in range(H) for g in range(ng)])


@pytest.mark.parametrize("e", [-70, 60])
def test_builder_extreme_magnitudes(e):
    """Samples scaled by 2^e (exact in bf16): at 2^-70 the encoder's float32 products fall
    below the normal range, at 2^60 its squared norms reach float32 overflow; the
    assignment must still be the float64 nearest center, so the books stay bit-exact."""
    T, Tc, G, S, H, d, n_iter = 4, 2, 16, 400, 1, 64, 3
    print(f"\ncase build extreme magnitudes x 2^{e}", flush=True)
    bits, rng = _samples(63, T, S, H, d)
    bits = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(bits) * np.float32(2.0 ** e))
    assert np.isfinite(synth.bf16_bits_to_f32(bits)).all()
    nblk, ng = T // Tc, d // (G // Tc)
    draws = rng.random((nblk, H, ng, 256))
    out = _gpu_build(bits, draws, 0, T, Tc, G, n_iter)
    ref = orc.build_codebooks(bits, draws, Tc, G, n_iter)
    _compare(out[:, 0], ref, [(b, h, g) for b in range(nblk) for h in range(H) for g in range(ng)])


def test_builder_few_samples_and_v_half():
    """S < 256: the seeding runs out of distinct samples (every D^2 reaches 0 and the uniform
    fallback repeats samples); only the selected half (V) is written."""
    T, Tc, G, S, H, d = 4, 2, 16, 100, 1, 64
    print("\ncase build few samples", flush=True)
    bits, rng = _samples(62, T, S, H, d)
    draws = rng.random((2, H, 8, 256))
    pre = np.full((2, 2, H, 8, Tc, 256, 8), 0x1234, dtype=np.uint16)
    out = _gpu_build(bits, draws, 1, T, Tc, G, 3, codebooks=pre)
    assert (out[:, 0] == 0x1234).all()
    ref = orc.build_codebooks(bits, draws, Tc, G, 3)
    _compare(out[:, 1], ref, [(b, 0, g) for b in range(2) for g in range(8)])


def test_builder_ouro_shape_sampled_books():
    """Ouro-shaped layer: 16 heads, d = 128, T = Tc = 4, G = 32, 4096 samples, 10 Lloyd
    iterations; every book is built on the GPU, three are checked against the oracle."""
    T, Tc, G, S, H, d = 4, 4, 32, 4096, 16, 128
    print("\ncase build Ouro shape", flush=True)
    bits, rng = _samples(63, T, S, H, d)
    draws = rng.random((1, H, 16, 256))
    out = _gpu_build(bits, draws, 0, T, Tc, G, 10)
    books = [(0, 0, 0), (0, 7, 11), (0, 15, 3)]
    ref = orc.build_codebooks(bits, draws, Tc, G, 10, books=books)
    _compare(out[:, 0], ref, books)
    # every book has 256 codewords drawn from a non-degenerate training set
    assert np.all(out[:, 0] != 0x7FC0)


@pytest.mark.parametrize("T,Tc,G,S,H,d,n_iter", [
    (4, 2, 16, 600, 2, 64, 3),
    (4, 4, 32, 700, 1, 128, 2),
])
def test_weighted_builder_matches_oracle(T, Tc, G, S, H, d, n_iter):
    """Per-vector weights (a quarter of them 0, the rest spread over two decades)."""
    print(f"\ncase weighted build T={T} Tc={Tc} G={G} S={S} H={H} d={d}", flush=True)
    bits, rng = _samples(64, T, S, H, d)
    nblk, ng = T // Tc, d // (G // Tc)
    draws = rng.random((nblk, H, ng, 256))
    w = 10.0 ** rng.uniform(-1, 1, (nblk, S, H, ng))
    w[rng.random(w.shape) < 0.25] = 0.0
    out = _gpu_build(bits, draws, 1, T, Tc, G, n_iter, weights=w)
    ref = orc.build_codebooks(bits, draws, Tc, G, n_iter, weights=w)
    _compare(out[:, 1], ref, [(b, h, g) for b in range(nblk) for h in range(H) for g in range(ng)])


def test_weighted_builder_degenerate_weights():
    """Books whose weights leave the seeding's corner rules in charge: all weights 0 (no
    positive total: every draw takes floor(u S)), a single positive weight, three positive
    weights (fewer than the 256 codes, so the D^2 terms run out), and one weight a million
    times the others; the remaining books carry ordinary weights."""
    T, Tc, G, S, H, d = 4, 2, 16, 300, 1, 64
    print("\ncase weighted build, degenerate weights", flush=True)
    bits, rng = _samples(67, T, S, H, d)
    nblk, ng = T // Tc, d // (G // Tc)
    draws = rng.random((nblk, H, ng, 256))
    w = 10.0 ** rng.uniform(-1, 1, (nblk, S, H, ng))
    w[0, :, 0, 0] = 0.0
    w[0, :, 0, 1] = 0.0
    w[0, 17, 0, 1] = 2.5
    w[0, :, 0, 2] = 0.0
    w[0, [5, 150, 299], 0, 2] = [1.0, 0.5, 3.0]
    w[1, :, 0, 3] = 1.0
    w[1, 42, 0, 3] = 1e6
    out = _gpu_build(bits, draws, 0, T, Tc, G, 3, weights=w)
    ref = orc.build_codebooks(bits, draws, Tc, G, 3, weights=w)
    _compare(out[:, 0], ref, [(b, h, g) for b in range(nblk) for h in range(H) for g in range(ng)])


def test_builder_at_the_lds_seeding_limit():
    """S = 8192, the largest count whose seeding keeps D^2 and running sums in LDS."""
    T, Tc, G, S, H, d = 4, 4, 32, 8192, 1, 64
    print("\ncase build S=8192", flush=True)
    bits, rng = _samples(66, T, S, H, d)
    draws = rng.random((1, H, 8, 256))
    out = _gpu_build(bits, draws, 0, T, Tc, G, 2)
    books = [(0, 0, 0), (0, 0, 5)]
    _compare(out[:, 0], orc.build_codebooks(bits, draws, Tc, G, 2, books=books), books)


@pytest.mark.parametrize("Tc,G,S,weighted", [(4, 32, 32768, False), (2, 16, 8200, True)])
def test_builder_at_calibration_scale(Tc, G, S, weighted):
    """S = 32768 sample tokens per book (16 calibration sequences of 2048 tokens), above
    the LDS seeding limit (D^2 in the workspace), Ouro-shaped layer (16 heads, d = 128),
    10 Lloyd iterations; sampled books bit-exact against the oracle.  A weighted case
    just above the limit covers the weighted terms of that path."""
    import time
    T, H, d = 4, 16, 128
    nblk, ng = T // Tc, d // (G // Tc)
    print(f"\ncase build calibration scale Tc={Tc} G={G} S={S} weighted={weighted}", flush=True)
    bits, rng = _samples(67, T, S, H, d)
    draws = rng.random((nblk, H, ng, 256))
    w = None
    if weighted:
        w = 10.0 ** rng.uniform(-1, 1, (nblk, S, H, ng))
        w[rng.random(w.shape) < 0.25] = 0.0
    _gpu_build(bits, draws, 0, T, Tc, G, 1, weights=w)    # warm-up
    t0 = time.perf_counter()
    out = _gpu_build(bits, draws, 0, T, Tc, G, 10, weights=w)
    dt = time.perf_counter() - t0
    import parity_log as plog
    plog.case(f"codebook builder at calibration scale: Tc={Tc} G={G} S={S} weighted={weighted}, "
              f"{nblk * H * ng} books, 10 Lloyd iterations")
    plog.line(f"build time {dt * 1e3:.1f} ms (host-timed, one call); sampled books {books_desc(nblk, ng)} "
              f"compared bit for bit below")
    books = [(0, 0, 0), (nblk - 1, 9, ng - 1)]
    ref = orc.build_codebooks(bits, draws, Tc, G, 10, books=books, weights=w)
    _compare(out[:, 0], ref, books)
    plog.line(f"books {books}: bit-exact against the oracle")


def test_weighted_builder_unit_weights_is_unweighted():
    T, Tc, G, S, H, d = 4, 4, 32, 4096, 16, 128
    print("\ncase unit weights Ouro shape", flush=True)
    bits, rng = _samples(65, T, S, H, d)
    draws = rng.random((1, H, 16, 256))
    a = _gpu_build(bits, draws, 0, T, Tc, G, 4)
    b = _gpu_build(bits, draws, 0, T, Tc, G, 4, weights=np.ones((1, S, H, 16)))
    assert (a == b).all()


def test_builder_rejects_bad_arguments():
    import sub_bit_loop_amd as lvq
    dev = torch.device("cuda:0")
    x = torch.zeros((4, 16, 1, 64), dtype=torch.bfloat16, device=dev)
    u = torch.zeros((2, 1, 8, 256), dtype=torch.float64, device=dev)
    with pytest.raises(lvq.LvqError):
        lvq.lvq_build_codebooks(x, u, 2, 4, 2, 16, 1)            # kv_sel
    with pytest.raises(lvq.LvqError):
        lvq.lvq_build_codebooks(x, u, 0, 4, 2, 16, -1)           # n_iter
    with pytest.raises(ValueError):
        lvq.lvq_build_codebooks(x, u, 0, 4, 2, 16, 1,
                                weights=torch.ones((2, 15, 1, 8), dtype=torch.float64, device=dev))
    big = torch.zeros((4, 32769, 1, 64), dtype=torch.bfloat16, device=dev)
    with pytest.raises(lvq.LvqError):
        lvq.lvq_build_codebooks(big, u, 0, 4, 2, 16, 1)          # S above 32768
