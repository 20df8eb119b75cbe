"""The benchmark's algorithmic byte and flop models (the numerators of its roofline
figures) reproduce the per-call workload figures derived independently from the
method: index rows of every coded token, bf16 sink and recent tokens, the step-t
codebook slices once, and 7 d flops per cached (token, head).  No GPU needed."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402  (the module imports torch only inside main())


def test_decode_call_bytes_at_the_ouro_shape():
    q_end = bench.synth_q_end()
    assert q_end == 32704                          # 8 * floor((32768 - 64) / 8)
    coded = q_end - bench.N_SINK                   # 32700 coded tokens per sequence
    ng = bench.D // (bench.G // bench.TC)          # 16 groups
    idx = bench.B * coded * bench.H * 2 * ng       # one byte per (token, head, group, K/V)
    bf = bench.B * (bench.N_SINK + bench.L - q_end) * bench.H * 2 * bench.D * 2
    books = bench.H * 2 * 256 * bench.D * 2
    assert idx == pytest.approx(133.94e6, rel=1e-4)
    assert bf == pytest.approx(4.46e6, rel=1e-3)
    assert books == pytest.approx(2.10e6, rel=1e-2)
    total = bench.algorithmic_bytes_per_call(q_end)
    assert total == pytest.approx(140.7e6, rel=1e-3)
    assert 0 < total - (idx + bf + books) < 0.3e6   # query, output, lse and page ids


def test_decode_call_flops_at_the_ouro_shape():
    # per (token, head): d/2 pairs rotated (6 flops each), q.k (2 d), p.v (2 d)
    per = (bench.D // 2) * 6 + 2 * bench.D + 2 * bench.D
    assert per == 7 * bench.D == 896
    assert bench.algorithmic_flops_per_call() == bench.B * bench.H * bench.L * per
    assert bench.algorithmic_flops_per_call() == pytest.approx(3.758e9, rel=1e-3)


def test_more_than_one_gpu_is_refused_with_a_message():
    """The library has no multi-GPU path: --gpus N > 1 exits at once (no GPU touched)."""
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_valu_floor_at_the_ouro_shape():
    """512 float32 lane operations per cached (token, head) at d = 128 (6 per channel pair
    for the rotated score, one FMA per channel for the value sum) over 4.19 M (token, head)
    at 256 CUs x 64 lanes x 2.4 GHz: 54.6 us."""
    assert bench.VALU_OPS_PER_TOKEN_HEAD == 512
    assert bench.valu_floor_us() == pytest.approx(54.6, abs=0.05)


def test_cpu_baseline_worker_runs_every_pair_of_a_small_call(tmp_path):
    """The CPU baseline's worker (a child process with forked oracle workers, no GPU)
    covers every (b, head) pair of a saved call and reports its cores."""
    import numpy as np
    from cachebuild import build_cache
    c = build_cache(41, 2, [200, 77], 2, 64, 4, 2, 16, 4, 16, books="random", index="random")
    t = 1
    arrays = dict(ip=c.index_pages, bp=c.bf16_pages, cb=c.codebooks, q=c.q[t], pt=c.page_table,
                  bt=c.bf16_table, pos=c.seq_len, qe=c.q_end,
                  meta=np.array([c.B, c.H, c.d, c.T, c.Tc, c.G, c.n_sink, t]))
    for k, v in arrays.items():
        np.save(tmp_path / f"{k}.npy", np.ascontiguousarray(v))
    w = bench.cpu_worker(str(tmp_path), 2, 60.0)
    assert w["pairs"] == w["of"] == c.B * c.H
    assert w["cores"] == 2 and w["seconds"] > 0
    assert bench.host_cores(0) >= 1 and bench.host_cores(100) <= 16
    assert isinstance(bench.cpu_model(), str)
