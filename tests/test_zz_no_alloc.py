"""lvq_decode_attn_noalloc (no workspace: the library's fixed device scratch array) against
lvq_decode_attn with a caller workspace, through the C ABI.  Same kernels, so the outputs
must be bit-identical; one case is also checked against the oracle.  Several calls run in
a row with different sizes (a smaller input after a larger one, then the larger again), on
the grouped (2 query heads per KV head), per-head (d = 64) and multi-row (8 query heads
per KV head) routes, so stale scratch contents can never leak."""
import numpy as np
import pytest
import torch

from cachebuild import build_cache
from gpu_helpers import attn_close, shape_of, to_dev

pytestmark = pytest.mark.gpu


def _both(dc, t):
    import sub_bit_loop_amd as lvq
    shp = shape_of(dc)
    args = (dc.q[t].contiguous(), dc.page_table, dc.index_pages, dc.bf16_pages, dc.bf16_table, dc.codebooks,
            t, dc.pos, dc.seq_len, dc.q_end, dc.rope, shp)
    B, Hq, d = dc.q.shape[1], dc.q.shape[2], dc.q.shape[3]
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
    lvq.lvq_decode_attn_noalloc(*args, out, lse)
    ref_out, ref_lse = lvq.lvq_decode_attn(*args)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy(), ref_out.cpu().numpy(), ref_lse.cpu().numpy()


def _same(a, b):
    np.testing.assert_array_equal(a[0], a[2])
    np.testing.assert_array_equal(a[1], a[3])
    if b is not None:
        np.testing.assert_array_equal(a[0], b[0])
        np.testing.assert_array_equal(a[1], b[1])


def test_noalloc_matches_the_workspace_entry_point():
    print("\ncase lvq_decode_attn_noalloc: large, small, large again; grouped, per-head and multi-row routes",
          flush=True)
    big = to_dev(build_cache(61, 4, [3000, 2500, 1200, 900], 4, 128, 4, 4, 32, 4, 64, Hq=8,
                             books="random", index="random"))   # 2 query heads per KV head: grouped route
    small = build_cache(62, 2, [300, 101], 2, 64, 4, 2, 16, 4, 16, books="random", index="random")
    small_d = to_dev(small)
    wide = to_dev(build_cache(63, 2, [700, 1500], 1, 128, 4, 4, 32, 4, 64, Hq=8,
                              books="random", index="random"))   # 8 query heads per KV head: multi-row route
    r_big = _both(big, 1)
    _same(r_big, None)
    r_small = _both(small_d, 3)                                  # a smaller input second
    _same(r_small, None)
    ro, rl = small.oracle_attn(3)
    ok, mabs, mrel = attn_close(r_small[0], ro)
    assert ok, f"max-abs {mabs:.3e} max-rel {mrel:.3e}"
    assert np.abs(r_small[1] - rl).max() <= 1e-4
    _same(_both(big, 1), r_big)                                  # the larger input again
    r_wide = _both(wide, 2)
    _same(r_wide, None)
    _same(_both(small_d, 3), r_small)
    print(f"  bit-identical to lvq_decode_attn on every call; small case vs oracle max-abs {mabs:.2e}", flush=True)
