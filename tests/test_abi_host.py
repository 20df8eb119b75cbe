"""The C-ABI library loads, exports every declared entry point, and rejects bad
arguments on the host before touching a device (no GPU needed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lvq.h")


@pytest.fixture(scope="module")
def L():
    from sub_bit_loop_amd import _abi
    if not os.path.exists(_abi.LIB_PATH):
        from sub_bit_loop_amd import build
        build.build()
    return _abi.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lvq_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), f"{n} declared in lvq.h but not exported"
    from sub_bit_loop_amd import _abi
    assert sorted(_abi.EXPORTS) == names


def test_version_and_error_text(L):
    assert L.lvq_version() == 1
    assert isinstance(L.lvq_last_error(), bytes)


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first
NUL = ctypes.c_void_p(0)


def enc(L, kv=FAKE, cb=FAKE, sel=0, T=4, Tc=2, G=16, N=8, H=1, d=64, out=FAKE):
    return L.lvq_encode(kv, cb, sel, T, Tc, G, N, H, d, out, NUL)


def test_encode_validation(L):
    assert enc(L, kv=NUL) == 1
    assert enc(L, out=NUL) == 1
    assert enc(L, Tc=3) == 1                     # Tc does not divide T
    assert enc(L, T=6, Tc=3, G=16) == 1          # Tc does not divide G
    assert enc(L, G=24, Tc=2, d=64, T=4) == 1    # c = 12 does not divide 64
    assert enc(L, sel=2) == 1
    assert enc(L, N=-1) == 1
    assert enc(L, d=96, G=16, Tc=2) == 2         # valid but not compiled
    assert enc(L, G=64, Tc=2) == 2
    assert b"Tc" in L.lvq_last_error() or L.lvq_last_error()
    assert enc(L, N=0) == 0                      # empty input is a no-op
    # pages: N must be a multiple of 8
    assert L.lvq_encode_pages(FAKE, FAKE, 0, 4, 2, 16, 12, 1, 64, FAKE, 4, FAKE, NUL) == 1
    assert L.lvq_reencode_pages(FAKE, FAKE, FAKE, -1, FAKE, 4, 2, 16, 1, 64, 4, 4, FAKE, NUL) == 1
    assert L.lvq_reencode_pages(FAKE, FAKE, FAKE, 0, FAKE, 4, 2, 16, 1, 64, 4, 4, FAKE, NUL) == 0


def test_reencode_layers_validation(L):
    from sub_bit_loop_amd import _abi
    tab = (_abi.ReencodeLayer * 2)()
    tab[0] = _abi.ReencodeLayer(FAKE, FAKE, FAKE, 4, 4)
    tab[1] = _abi.ReencodeLayer(FAKE, FAKE, FAKE, 4, 4)
    args = (FAKE, FAKE, 3, 4, 2, 16, 1, 64, NUL)
    assert L.lvq_reencode_pages_layers(tab, -1, *args) == 1
    assert L.lvq_reencode_pages_layers(None, 2, *args) == 1
    assert L.lvq_reencode_pages_layers(tab, 2, FAKE, FAKE, -1, 4, 2, 16, 1, 64, NUL) == 1
    assert L.lvq_reencode_pages_layers(tab, 2, NUL, FAKE, 3, 4, 2, 16, 1, 64, NUL) == 1
    assert L.lvq_reencode_pages_layers(tab, 2, FAKE, FAKE, 3, 4, 3, 16, 1, 64, NUL) == 1   # Tc does not divide T
    tab[1] = _abi.ReencodeLayer(FAKE, NUL, FAKE, 4, 4)                                      # second layer bad
    assert L.lvq_reencode_pages_layers(tab, 2, *args) == 1
    tab[1] = _abi.ReencodeLayer(FAKE, FAKE, NUL, 4, 4)
    assert L.lvq_reencode_pages_layers(tab, 2, *args) == 1
    tab[1] = _abi.ReencodeLayer(FAKE, FAKE, FAKE, -1, 4)
    assert L.lvq_reencode_pages_layers(tab, 2, *args) == 1
    assert b"layer 1" in L.lvq_last_error()
    tab[1] = _abi.ReencodeLayer(FAKE, FAKE, FAKE, 4, 4)
    assert L.lvq_reencode_pages_layers(tab, 0, *args) == 0                                  # no layers: no-op
    assert L.lvq_reencode_pages_layers(tab, 2, FAKE, FAKE, 0, 4, 2, 16, 1, 64, NUL) == 0    # no pages: no-op


def test_rope_table_sizes(L):
    assert L.lvq_rope_table_bytes(512, 64) == (32 + 16) * 32 * 2 * 4 + 32 * 8
    assert L.lvq_rope_table_bytes(513, 64) == (33 + 16) * 32 * 2 * 4 + 32 * 8
    assert L.lvq_rope_table_bytes(0, 64) == 0
    assert L.lvq_rope_tables(512, 64, ctypes.c_double(10000.0), FAKE, 10, NUL) == 3
    assert L.lvq_rope_tables(512, 63, ctypes.c_double(10000.0), FAKE, 1 << 20, NUL) == 1
    assert L.lvq_rope_tables(512, 64, ctypes.c_double(1.0), FAKE, 1 << 20, NUL) == 1


def shape(**kw):
    from sub_bit_loop_amd import _abi
    base = dict(B=2, H=2, Hq=4, d=128, T=4, Tc=4, G=32, n_sink=4, max_pages=64, bf16_row=12,
                n_index_pages=100, n_bf16_pages=20, max_seq_len=512, rope_max_len=513,
                n_splits=0, scale=0.0)
    base.update(kw)
    return _abi.make_shape(**base)


def attn(L, shp, t=0, ws_bytes=1 << 30, q=FAKE):
    return L.lvq_decode_attn(q, FAKE, FAKE, FAKE, FAKE, FAKE, t, FAKE, FAKE, FAKE, FAKE,
                             ctypes.byref(shp), FAKE, NUL, FAKE, ws_bytes, NUL)


def test_attn_validation(L):
    assert attn(L, shape(), q=NUL) == 1
    assert attn(L, shape(), t=4) == 1
    assert attn(L, shape(Hq=3)) == 1
    assert attn(L, shape(Tc=3)) == 1
    assert attn(L, shape(n_sink=9)) == 1
    assert attn(L, shape(max_pages=10)) == 1
    assert attn(L, shape(rope_max_len=512)) == 1
    assert attn(L, shape(n_index_pages=0)) == 1   # an all-bf16 cache still passes one coded page
    assert attn(L, shape(n_bf16_pages=0)) == 1
    assert attn(L, shape(d=96, G=16, Tc=2)) == 2
    assert attn(L, shape(G=16, Tc=4)) == 2       # c = 4 not compiled for decode
    assert attn(L, shape(d=64, G=32, Tc=1)) == 2  # c = 32 at d = 64 not compiled
    assert attn(L, shape(), ws_bytes=4) == 3
    assert L.lvq_decode_scores(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, FAKE, FAKE, FAKE,
                               ctypes.byref(shape()), FAKE, NUL, NUL, FAKE, 1 << 30, NUL) == 1


def test_workspace_size_covers_every_split(L):
    """Records [Hq][W + B][d + 2] float32 and the tile table [B + 1] int32, W waves per head
    in whole workgroups of 12: W = 12 * ceil(n_splits / 12), or automatically 256 / Hq
    workgroups per head, capped at about 4 tiles per wave of the largest work list."""
    from sub_bit_loop_amd import _abi
    for B, Hq, msl, ns, W in ((8, 16, 32768, 0, 192), (1, 16, 65536, 0, 192), (64, 16, 16384, 0, 192),
                              (1, 1, 512, 7, 12), (1, 1, 512, 0, 12), (2, 4, 100, 0, 12),
                              (1, 1, 1 << 20, 0, 3072), (3, 2, 4096, 1000, 1008)):
        s = shape(B=B, H=Hq, Hq=Hq, max_seq_len=msl, rope_max_len=msl + 1, max_pages=(msl + 7) // 8,
                  n_splits=ns)
        nbytes = _abi.lvq_decode_attn_workspace_bytes(s)
        assert nbytes == Hq * (W + B) * 130 * 4 + (B + 1) * 4, (B, Hq, msl, ns, nbytes)


def test_workspace_query_refuses_malformed_shapes(L):
    """The size query returns 0 (and does not divide by zero) for a shape the entry points
    would refuse: H or Tc zero, Hq not a multiple of H."""
    from sub_bit_loop_amd import _abi
    for kw in (dict(H=0), dict(H=-1), dict(Hq=3), dict(Tc=0), dict(G=0), dict(B=0), dict(max_seq_len=0)):
        assert _abi.lvq_decode_attn_workspace_bytes(shape(**kw)) == 0, kw
    assert _abi.lvq_decode_attn_workspace_bytes(shape()) > 0


def test_workspace_size_of_grouped_decode(L):
    """At 2 and 4 query heads per KV head (d = 128) the workspace holds the larger of the
    per-head records (lvq_decode_scores keeps that kernel) and the grouped kernel's: records
    [H][W + 4 B][g heads][d + 2] float32, W waves per KV head in whole workgroups of 16,
    automatically 256 / H workgroups per KV head capped at about 4 tiles per quad of the
    largest work list; then the tile table [B + 1] int32."""
    from sub_bit_loop_amd import _abi
    for B, H, g, msl, ns, Wg, Wph in ((8, 4, 4, 32768, 0, 1024, 192), (1, 4, 4, 65536, 0, 1024, 192),
                                      (2, 1, 4, 100, 0, 32, 12), (3, 2, 4, 4096, 1000, 1008, 1008),
                                      (8, 8, 2, 32768, 0, 512, 192)):
        Hq = g * H
        s = shape(B=B, H=H, Hq=Hq, max_seq_len=msl, rope_max_len=msl + 1, max_pages=(msl + 7) // 8,
                  n_splits=ns)
        grouped = H * (Wg + 4 * B) * g * 130 * 4 + (B + 1) * 4
        per_head = Hq * (Wph + B) * 130 * 4 + (B + 1) * 4
        nbytes = _abi.lvq_decode_attn_workspace_bytes(s)
        assert nbytes == max(grouped, per_head), (B, H, msl, ns, nbytes, grouped, per_head)


def test_workspace_size_of_multi_row_decode(L):
    """At 8 and 16 query heads per KV head (d = 128) lvq_decode_attn runs on the multi-row
    kernel: the workspace holds the larger of the per-head records and the multi-row
    kernel's, records [H][W + B][16 rows][d + 2] float32 and first units [B + 1] int32 (one
    16-row block per KV head), W waves per KV head in whole workgroups of 8: automatically
    256 / H workgroups capped at about 4 tiles per wave of the largest work list
    (B * (max_seq_len / 16 + 4) tiles)."""
    from sub_bit_loop_amd import _abi
    for B, H, g, msl, ns, Wr, Wph in ((8, 2, 8, 32768, 0, 1024, 192), (8, 1, 16, 32768, 0, 2048, 192),
                                      (2, 1, 8, 100, 0, 8, 12), (3, 2, 8, 4096, 100, 104, 108)):
        Hq = g * H
        s = shape(B=B, H=H, Hq=Hq, max_seq_len=msl, rope_max_len=msl + 1, max_pages=(msl + 7) // 8,
                  n_splits=ns)
        rows = H * (Wr + B) * 16 * 130 * 4 + (B + 1) * 4
        per_head = Hq * (Wph + B) * 130 * 4 + (B + 1) * 4
        nbytes = _abi.lvq_decode_attn_workspace_bytes(s)
        assert nbytes == max(rows, per_head), (B, H, g, msl, ns, nbytes, rows, per_head)


def test_builder_validation(L):
    ws = FAKE
    # a null weights pointer is fine (unweighted); the rest must be given
    assert L.lvq_build_codebooks(NUL, FAKE, NUL, 0, 4, 2, 16, 100, 1, 64, 1, FAKE, ws, 1 << 30, NUL) == 1
    assert L.lvq_build_codebooks(FAKE, NUL, NUL, 0, 4, 2, 16, 100, 1, 64, 1, FAKE, ws, 1 << 30, NUL) == 1
    assert L.lvq_build_codebooks(FAKE, FAKE, NUL, 2, 4, 2, 16, 100, 1, 64, 1, FAKE, ws, 1 << 30, NUL) == 1
    assert L.lvq_build_codebooks(FAKE, FAKE, NUL, 0, 4, 2, 16, 0, 1, 64, 1, FAKE, ws, 1 << 30, NUL) == 1
    assert L.lvq_build_codebooks(FAKE, FAKE, NUL, 0, 4, 2, 16, 32769, 1, 64, 1, FAKE, ws, 1 << 30, NUL) == 2
    # above the LDS seeding limit the workspace also holds one float64 D^2 per (book, sample)
    small = L.lvq_build_codebooks_workspace_bytes(4, 2, 16, 8192, 1, 64)
    big = L.lvq_build_codebooks_workspace_bytes(4, 2, 16, 8200, 1, 64)
    assert big - small >= 2 * 8 * 8224 * 8
    assert L.lvq_build_codebooks(FAKE, FAKE, NUL, 0, 4, 2, 16, 100, 1, 64, 1001, FAKE, ws, 1 << 30, NUL) == 1
    need = L.lvq_build_codebooks_workspace_bytes(4, 2, 16, 100, 1, 64)
    # centers (2 blocks x 8 groups x 256 x 16 float64, 256-aligned) + assignments
    assert need == 2 * 8 * 256 * 16 * 8 + 2 * 100 * 8
    assert L.lvq_build_codebooks(FAKE, FAKE, NUL, 0, 4, 2, 16, 100, 1, 64, 1, FAKE, ws, need - 1, NUL) == 3


def test_cache_descriptor_validation(L):
    from sub_bit_loop_amd import _abi
    assert L.lvq_cache_min_bf16_row(64) == 10
    assert L.lvq_cache_min_bf16_row(0) == 2
    assert L.lvq_cache_min_bf16_row(5) == 3
    ptrs = [0x1000] * 9

    def desc(**kw):
        base = dict(B=2, max_pages=16, bf16_row=10, n_sink=4, n_recent=64, n_index_pages=8, n_bf16_pages=8)
        base.update(kw)
        return _abi.CacheDesc(*base.values(), *ptrs)

    assert L.lvq_cache_init(None, NUL) == 1
    for bad in (dict(n_sink=9), dict(bf16_row=9), dict(B=0), dict(n_index_pages=0), dict(n_recent=-1)):
        assert L.lvq_cache_init(ctypes.byref(desc(**bad)), NUL) == 1, bad
    d = desc()
    assert L.lvq_cache_prefill(ctypes.byref(d), NUL, NUL) == 1
    assert L.lvq_cache_release(ctypes.byref(d), NUL, NUL) == 1
    assert L.lvq_cache_store_tokens(ctypes.byref(d), 2, 0, 1, FAKE, FAKE, 4, 1, 64, FAKE, NUL) == 1   # b = B
    assert L.lvq_cache_store_tokens(ctypes.byref(d), 0, 0, 0, FAKE, FAKE, 4, 1, 64, FAKE, NUL) == 0   # nothing
    assert L.lvq_cache_store_tokens(ctypes.byref(d), 0, 0, 1, FAKE, FAKE, 4, 1, 60, FAKE, NUL) == 1   # d % 8
    assert L.lvq_cache_append(ctypes.byref(d), 3, 2, FAKE, FAKE, 4, 1, 64, FAKE, NUL) == 1           # steps 3..4
    assert L.lvq_cache_append(ctypes.byref(d), 0, 1, NUL, FAKE, 4, 1, 64, FAKE, NUL) == 1


def test_rows_shape_validation(L):
    from sub_bit_loop_amd import _abi

    def rs(**kw):
        base = dict(B=1, NQ=4, H=2, Hq=4, d=128, T=4, Tc=4, G=32, n_sink=4, max_pages=64, bf16_row=12,
                    n_index_pages=100, n_bf16_pages=20, max_prefix=500, rope_max_len=504, n_splits=0)
        base.update(kw)
        return _abi.RowsShape(*base.values(), 0.0)

    def call(s, k=FAKE, v=FAKE, ws_bytes=1 << 30):
        return L.lvq_rows_attn(FAKE, k, v, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, FAKE, FAKE, FAKE,
                               ctypes.byref(s), FAKE, FAKE, FAKE, ws_bytes, NUL)

    assert call(rs(), k=NUL) == 1                       # k_new without v_new
    assert call(rs(Hq=3)) == 1
    assert call(rs(rope_max_len=503)) == 1              # below max_prefix + NQ
    assert call(rs(max_pages=62)) == 1                  # 62 pages hold fewer than 500 tokens
    assert call(rs(n_index_pages=0)) == 1               # coded pool must hold a page
    assert call(rs(d=64, G=16, Tc=2)) == 2              # multi-row kernel compiled for d = 128 only
    need = L.lvq_rows_attn_workspace_bytes(ctypes.byref(rs()))
    # records [H * row blocks][W + B][16 rows][d + 2] float32 + first units [row blocks][B + 1]:
    # 1 row block (4 queries x 2 heads per KV head), W = 16 waves (2 workgroups: about 4
    # units per wave of 32 coded + 16 virtual units)
    assert need == 2 * 1 * (16 + 1) * 16 * 130 * 4 + 1 * 2 * 4
    assert call(rs(), ws_bytes=need - 1) == 3


def test_binding_shape_helpers():
    """The binding derives the shapes the kernels index by from the call's sizes, and
    refuses other tensors before anything is launched."""
    import torch
    from sub_bit_loop_amd import _abi
    assert _abi._coded_dims(4, 4, 32, 128) == (1, 16, 8)
    assert _abi._coded_dims(4, 2, 16, 64) == (2, 8, 8)
    assert _abi._coded_dims(4, 3, 32, 128) is None      # Tc does not divide T: the library rejects
    assert _abi._coded_dims(4, 0, 32, 128) is None
    assert _abi._book_shape(4, 2, 16, 3, 64) == (2, 2, 3, 8, 2, 256, 8)
    assert _abi._index_pool_shape(7, 8, 4, 32, 2, 128) == (7, 2, 2, 2, 8, 16)
    _abi._expect(torch.zeros(2, 3), "x", (2, 3))
    _abi._expect(torch.zeros(2, 3), "x", None)
    with pytest.raises(ValueError, match="needs"):
        _abi._expect(torch.zeros(2, 3), "x", (3, 2))


def test_noalloc_refuses_shapes_beyond_its_scratch(L):
    """lvq_decode_attn_noalloc refuses, before touching a device, a shape whose partial
    records exceed the fixed scratch array (LVQ_ENOSPC), and reports invalid shapes as the
    workspace entry point does."""
    big = shape(B=4096, Hq=64, H=64)
    assert L.lvq_decode_attn_workspace_bytes(ctypes.byref(big)) > 32 << 20
    rc = L.lvq_decode_attn_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, FAKE, FAKE, FAKE,
                                   ctypes.byref(big), FAKE, NUL, NUL)
    assert rc == 3 and b"scratch" in L.lvq_last_error()
