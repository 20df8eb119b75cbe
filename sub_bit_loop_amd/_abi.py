"""ctypes binding of liblvq.so (include/lvq.h).

Argument marshalling only: tensors are checked for device, dtype and layout,
and their data pointers and the current HIP stream are handed to the C ABI.
Every step of the hot path runs in the library's kernels; there is no fallback,
and a missing library raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblvq.so")

LVQ_OK, LVQ_EINVAL, LVQ_EUNSUPPORTED, LVQ_ENOSPC, LVQ_EDEVICE = range(5)
PAGE = 8
NCODES = 256

_i32, _f32, _f64, _sz, _vp = ctypes.c_int32, ctypes.c_float, ctypes.c_double, ctypes.c_size_t, ctypes.c_void_p


class LvqError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"lvq status {status}: {msg}")
        self.status = status


class AttnShape(ctypes.Structure):
    """Mirror of lvq_attn_shape."""
    _fields_ = [(n, _i32) for n in ("B", "H", "Hq", "d", "T", "Tc", "G", "n_sink", "max_pages",
                                   "bf16_row", "n_index_pages", "n_bf16_pages", "max_seq_len",
                                   "rope_max_len", "n_splits")] + [("scale", _f32), ("rejected", _vp)]


class RowsShape(ctypes.Structure):
    """Mirror of lvq_rows_shape."""
    _fields_ = [(n, _i32) for n in ("B", "NQ", "H", "Hq", "d", "T", "Tc", "G", "n_sink", "max_pages",
                                   "bf16_row", "n_index_pages", "n_bf16_pages", "max_prefix",
                                   "rope_max_len", "n_splits")] + [("scale", _f32), ("rejected", _vp)]


class CacheDesc(ctypes.Structure):
    """Mirror of lvq_cache."""
    _fields_ = [(n, _i32) for n in ("B", "max_pages", "bf16_row", "n_sink", "n_recent", "n_index_pages",
                                   "n_bf16_pages")] + \
               [(n, _vp) for n in ("page_table", "bf16_table", "seq_len", "q_end", "index_free", "bf16_free",
                                   "counters", "re_src", "re_dst")]


class ReencodeLayer(ctypes.Structure):
    """Mirror of lvq_reencode_layer."""
    _fields_ = [("bf16_pages", _vp), ("codebooks", _vp), ("index_pages", _vp), ("n_bf16_pages", _i32),
                ("n_index_pages", _i32)]


_CP = ctypes.POINTER(CacheDesc)

_SIGS = {
    "lvq_version": (_i32, []),
    "lvq_last_error": (ctypes.c_char_p, []),
    "lvq_encode": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp]),
    "lvq_encode_pages": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _i32, _vp, _vp]),
    "lvq_reencode_pages": (_i32, [_vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp]),
    "lvq_reencode_pages_layers": (_i32, [ctypes.POINTER(ReencodeLayer), _i32, _vp, _vp, _i32, _i32, _i32,
                                         _i32, _i32, _i32, _vp]),
    "lvq_build_codebooks_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "lvq_build_codebooks": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp,
                                   _sz, _vp]),
    "lvq_rope_table_bytes": (_sz, [_i32, _i32]),
    "lvq_rope_tables": (_i32, [_i32, _i32, _f64, _vp, _sz, _vp]),
    "lvq_decode_attn_workspace_bytes": (_sz, [ctypes.POINTER(AttnShape)]),
    "lvq_decode_attn": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp,
                               ctypes.POINTER(AttnShape), _vp, _vp, _vp, _sz, _vp]),
    "lvq_decode_attn_noalloc": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp,
                                       ctypes.POINTER(AttnShape), _vp, _vp, _vp]),
    "lvq_decode_scores": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp,
                                 ctypes.POINTER(AttnShape), _vp, _vp, _vp, _vp, _sz, _vp]),
    "lvq_rows_attn_workspace_bytes": (_sz, [ctypes.POINTER(RowsShape)]),
    "lvq_rows_attn": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp,
                             ctypes.POINTER(RowsShape), _vp, _vp, _vp, _sz, _vp]),
    "lvq_cache_min_bf16_row": (_i32, [_i32]),
    "lvq_cache_init": (_i32, [_CP, _vp]),
    "lvq_cache_prefill": (_i32, [_CP, _vp, _vp]),
    "lvq_cache_store_tokens": (_i32, [_CP, _i32, _i32, _i32, _vp, _vp, _i32, _i32, _i32, _vp, _vp]),
    "lvq_cache_begin_token": (_i32, [_CP, _vp]),
    "lvq_cache_append": (_i32, [_CP, _i32, _i32, _vp, _vp, _i32, _i32, _i32, _vp, _vp]),
    "lvq_cache_end_token": (_i32, [_CP, _vp]),
    "lvq_cache_commit": (_i32, [_CP, _vp]),
    "lvq_cache_release": (_i32, [_CP, _vp, _vp]),
}
EXPORTS = tuple(_SIGS)

_LIB = None


def lib() -> ctypes.CDLL:
    """Load liblvq.so (built in-tree); raises if it is missing."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise LvqError(LVQ_EDEVICE, f"{LIB_PATH} is not built (run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def _check(status: int) -> None:
    if status != LVQ_OK:
        raise LvqError(status, lib().lvq_last_error().decode())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t: torch.Tensor | None):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _dev(t: torch.Tensor, name: str, dtypes, ndim: int | None = None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    return t


BF16 = (torch.bfloat16, torch.int16, torch.uint16)   # bf16 bit patterns
I32 = (torch.int32,)
U8 = (torch.uint8,)
F32 = (torch.float32,)


def _coded_dims(T: int, Tc: int, G: int, d: int):
    """(nblk, ng, c) of a valid (T, Tc, G, d), else None (the library then rejects the call)."""
    if min(T, Tc, G, d) <= 0 or T % Tc or G % Tc or d % (G // Tc):
        return None
    c = G // Tc
    return T // Tc, d // c, c


def _expect(t: torch.Tensor, name: str, shape) -> None:
    """The kernels index these arrays by the call's sizes: a tensor of another shape
    would be read or written out of bounds, so it is refused here."""
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, the call needs {tuple(shape)}")


def _book_shape(T: int, Tc: int, G: int, H: int, d: int):
    """[nblk][2][H][ng][Tc][256][c], or None for sizes the library rejects."""
    dims = _coded_dims(T, Tc, G, d)
    return None if dims is None else (dims[0], 2, H, dims[1], Tc, NCODES, dims[2])


def _index_pool_shape(P: int, T: int, Tc: int, G: int, H: int, d: int):
    """[P][nblk][H][2][8][ng], or None for sizes the library rejects."""
    dims = _coded_dims(T, Tc, G, d)
    return None if dims is None else (P, dims[0], H, 2, PAGE, dims[1])


def lvq_version() -> int:
    return lib().lvq_version()


def lvq_encode(kv, codebooks, kv_sel: int, T: int, Tc: int, G: int, idx=None) -> torch.Tensor:
    """kv bf16 [T][N][H][d], codebooks bf16 [nblk][2][H][ng][Tc][256][c] -> idx uint8 [nblk][N][H][ng]."""
    _dev(kv, "kv", BF16, 4)
    _dev(codebooks, "codebooks", BF16, 7)
    T_, N, H, d = kv.shape
    if T_ != T:
        raise ValueError("kv.shape[0] != T")
    c = G // Tc if Tc > 0 else 0
    ng = d // c if c > 0 else 0
    _expect(codebooks, "codebooks", _book_shape(T, Tc, G, H, d))
    if idx is None:
        idx = torch.empty((max(T // max(Tc, 1), 0), N, H, ng), dtype=torch.uint8, device=kv.device)
    _dev(idx, "idx", U8)
    dims = _coded_dims(T, Tc, G, d)
    _expect(idx, "idx", None if dims is None else (dims[0], N, H, dims[1]))
    _check(lib().lvq_encode(_ptr(kv), _ptr(codebooks), kv_sel, T, Tc, G, N, H, d, _ptr(idx), _stream(kv)))
    return idx


def lvq_encode_pages(kv, codebooks, kv_sel: int, T: int, Tc: int, G: int, chunk_page,
                     index_pages) -> torch.Tensor:
    """Encode kv [T][N][H][d] into index_pages [P][nblk][H][2][8][ng] at pages chunk_page [N/8]."""
    _dev(kv, "kv", BF16, 4)
    _dev(codebooks, "codebooks", BF16, 7)
    _dev(chunk_page, "chunk_page", I32, 1)
    _dev(index_pages, "index_pages", U8, 6)
    T_, N, H, d = kv.shape
    if T_ != T:
        raise ValueError("kv.shape[0] != T")
    if chunk_page.numel() * PAGE < N:
        raise ValueError("chunk_page too short")
    _expect(codebooks, "codebooks", _book_shape(T, Tc, G, H, d))
    _expect(index_pages, "index_pages", _index_pool_shape(index_pages.shape[0], T, Tc, G, H, d))
    _check(lib().lvq_encode_pages(_ptr(kv), _ptr(codebooks), kv_sel, T, Tc, G, N, H, d,
                                  _ptr(chunk_page), index_pages.shape[0], _ptr(index_pages),
                                  _stream(kv)))
    return index_pages


def lvq_reencode_pages(bf16_pages, src_pages, dst_pages, codebooks, T: int, Tc: int, G: int,
                       index_pages) -> torch.Tensor:
    """Encode whole bf16 pages src_pages[i] (all steps, heads, K and V) into coded pages dst_pages[i]."""
    _dev(bf16_pages, "bf16_pages", BF16, 6)
    _dev(src_pages, "src_pages", I32, 1)
    _dev(dst_pages, "dst_pages", I32, 1)
    _dev(codebooks, "codebooks", BF16, 7)
    _dev(index_pages, "index_pages", U8, 6)
    if src_pages.numel() != dst_pages.numel():
        raise ValueError("src_pages and dst_pages differ in length")
    _, T_, H, _, _, d = bf16_pages.shape
    _expect(bf16_pages, "bf16_pages", (bf16_pages.shape[0], T, H, 2, PAGE, d))
    _expect(codebooks, "codebooks", _book_shape(T, Tc, G, H, d))
    _expect(index_pages, "index_pages", _index_pool_shape(index_pages.shape[0], T, Tc, G, H, d))
    _check(lib().lvq_reencode_pages(_ptr(bf16_pages), _ptr(src_pages), _ptr(dst_pages),
                                    src_pages.numel(), _ptr(codebooks), T, Tc, G, H, d,
                                    bf16_pages.shape[0], index_pages.shape[0], _ptr(index_pages),
                                    _stream(bf16_pages)))
    return index_pages


def lvq_reencode_pages_layers(layers, src_pages, dst_pages, T: int, Tc: int, G: int) -> None:
    """lvq_reencode_pages for every (bf16_pages, codebooks, index_pages) triple in layers, in one launch."""
    _dev(src_pages, "src_pages", I32, 1)
    _dev(dst_pages, "dst_pages", I32, 1)
    if src_pages.numel() != dst_pages.numel():
        raise ValueError("src_pages and dst_pages differ in length")
    layers = list(layers)
    tab = (ReencodeLayer * max(1, len(layers)))()
    H = d = 0
    for i, (bp, cb, ip) in enumerate(layers):
        _dev(bp, "bf16_pages", BF16, 6)
        _dev(cb, "codebooks", BF16, 7)
        _dev(ip, "index_pages", U8, 6)
        if i == 0:
            _, _, H, _, _, d = bp.shape
        elif (bp.shape[2], bp.shape[5]) != (H, d):
            raise ValueError("layers differ in heads or head dimension")
        _expect(bp, f"layer {i} bf16_pages", (bp.shape[0], T, H, 2, PAGE, d))
        _expect(cb, f"layer {i} codebooks", _book_shape(T, Tc, G, H, d))
        _expect(ip, f"layer {i} index_pages", _index_pool_shape(ip.shape[0], T, Tc, G, H, d))
        tab[i] = ReencodeLayer(_ptr(bp), _ptr(cb), _ptr(ip), bp.shape[0], ip.shape[0])
    if not layers:
        return
    _check(lib().lvq_reencode_pages_layers(tab, len(layers), _ptr(src_pages), _ptr(dst_pages),
                                           src_pages.numel(), T, Tc, G, H, d, _stream(layers[0][0])))


def lvq_build_codebooks(samples, draws, kv_sel: int, T: int, Tc: int, G: int, n_iter: int,
                        codebooks=None, ws=None, weights=None) -> torch.Tensor:
    """k-means codebooks of one of K / V from samples bf16 [T][S][H][d], float64 draws
    [nblk][H][ng][256] and optional float64 weights [nblk][S][H][ng]; writes half kv_sel of
    codebooks bf16 [nblk][2][H][ng][Tc][256][c]."""
    _dev(samples, "samples", BF16, 4)
    _dev(draws, "draws", (torch.float64,), 4)
    T_, S, H, d = samples.shape
    if T_ != T:
        raise ValueError("samples.shape[0] != T")
    c = G // Tc if Tc > 0 else 0
    nblk = T // Tc if Tc > 0 else 0
    ng = d // c if c > 0 else 0
    if tuple(draws.shape) != (nblk, H, ng, NCODES):
        raise ValueError(f"draws must have shape {(nblk, H, ng, NCODES)}")
    if weights is not None:
        _dev(weights, "weights", (torch.float64,), 4)
        if tuple(weights.shape) != (nblk, S, H, ng):
            raise ValueError(f"weights must have shape {(nblk, S, H, ng)}")
    if codebooks is None:
        codebooks = torch.zeros((nblk, 2, H, ng, Tc, NCODES, c), dtype=torch.bfloat16, device=samples.device)
    _dev(codebooks, "codebooks", BF16, 7)
    _expect(codebooks, "codebooks", _book_shape(T, Tc, G, H, d))
    need = lib().lvq_build_codebooks_workspace_bytes(T, Tc, G, S, H, d)
    if ws is None:
        ws = torch.empty(max(need, 4), dtype=torch.uint8, device=samples.device)
    _check(lib().lvq_build_codebooks(_ptr(samples), _ptr(draws), None if weights is None else _ptr(weights),
                                     kv_sel, T, Tc, G, S, H, d, n_iter,
                                     _ptr(codebooks), _ptr(ws), ws.numel() * ws.element_size(),
                                     _stream(samples)))
    return codebooks


def lvq_rope_table_bytes(max_len: int, d: int) -> int:
    return lib().lvq_rope_table_bytes(max_len, d)


def lvq_rope_tables(max_len: int, d: int, base: float = 10000.0, device="cuda") -> torch.Tensor:
    n = lvq_rope_table_bytes(max_len, d)
    if n == 0:
        raise LvqError(LVQ_EINVAL, "invalid rope table size")
    tab = torch.empty(n // 4, dtype=torch.float32, device=device)
    _check(lib().lvq_rope_tables(max_len, d, float(base), _ptr(tab), n, _stream(tab)))
    return tab


def _counter_ptr(rejected):
    """Device address of an optional int32/uint32 counter tensor (one element), or None."""
    if rejected is None:
        return None
    _dev(rejected, "rejected", (torch.int32,), 1)
    if rejected.numel() < 1:
        raise ValueError("rejected must hold one element")
    return rejected.data_ptr()


def make_shape(B, H, Hq, d, T, Tc, G, n_sink, max_pages, bf16_row, n_index_pages, n_bf16_pages,
               max_seq_len, rope_max_len, n_splits=0, scale=0.0, rejected=None) -> AttnShape:
    """rejected: None, or a one-element int32 device tensor that the kernels add one to for
    every page-id lookup outside its pool (the caller zeroes it)."""
    return AttnShape(B, H, Hq, d, T, Tc, G, n_sink, max_pages, bf16_row, n_index_pages,
                     n_bf16_pages, max_seq_len, rope_max_len, n_splits, scale, _counter_ptr(rejected))


def lvq_decode_attn_workspace_bytes(shp: AttnShape) -> int:
    return lib().lvq_decode_attn_workspace_bytes(ctypes.byref(shp))


def _attn_call(fn, q, page_table, index_pages, bf16_pages, bf16_table, codebooks, t, pos, seq_len,
               q_end, rope_tab, shp: AttnShape, out, lse, ws, scores=None, noalloc=False):
    _dev(q, "q", BF16, 3)
    _dev(page_table, "page_table", I32, 2)
    _dev(index_pages, "index_pages", U8, 6)
    _dev(bf16_pages, "bf16_pages", BF16, 6)
    _dev(bf16_table, "bf16_table", I32, 2)
    _dev(codebooks, "codebooks", BF16, 7)
    for name, x in (("pos", pos), ("seq_len", seq_len), ("q_end", q_end)):
        _dev(x, name, I32, 1)
    _dev(rope_tab, "rope_tab", F32, 1)
    if tuple(page_table.shape) != (shp.B, shp.max_pages) or tuple(bf16_table.shape) != (shp.B, shp.bf16_row):
        raise ValueError("page_table / bf16_table do not match the shape")
    if index_pages.shape[0] != shp.n_index_pages or bf16_pages.shape[0] != shp.n_bf16_pages:
        raise ValueError("pool sizes do not match the shape")
    if rope_tab.numel() * 4 < lvq_rope_table_bytes(shp.rope_max_len, shp.d):
        raise ValueError("rope table too small")
    _expect(q, "q", (shp.B, shp.Hq, shp.d))
    for name, x in (("pos", pos), ("seq_len", seq_len), ("q_end", q_end)):
        _expect(x, name, (shp.B,))
    _expect(index_pages, "index_pages", _index_pool_shape(shp.n_index_pages, shp.T, shp.Tc, shp.G, shp.H, shp.d))
    _expect(bf16_pages, "bf16_pages", (shp.n_bf16_pages, shp.T, shp.H, 2, PAGE, shp.d))
    _expect(codebooks, "codebooks", _book_shape(shp.T, shp.Tc, shp.G, shp.H, shp.d))
    dev = q.device
    if out is None:
        out = torch.empty((shp.B, shp.Hq, shp.d), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((shp.B, shp.Hq), dtype=torch.float32, device=dev)
    if ws is None and not noalloc:
        ws = torch.empty(max(lvq_decode_attn_workspace_bytes(shp), 4), dtype=torch.uint8, device=dev)
    _dev(out, "out", F32)
    _dev(lse, "lse", F32)
    _expect(out, "out", (shp.B, shp.Hq, shp.d))
    _expect(lse, "lse", (shp.B, shp.Hq))
    args = [_ptr(q), _ptr(page_table), _ptr(index_pages), _ptr(bf16_pages), _ptr(bf16_table),
            _ptr(codebooks), int(t), _ptr(pos), _ptr(seq_len), _ptr(q_end), _ptr(rope_tab),
            ctypes.byref(shp), _ptr(out), _ptr(lse)]
    if scores is not None:
        _dev(scores, "scores", F32)
        _expect(scores, "scores", (shp.B, shp.Hq, shp.max_seq_len))
        args.append(_ptr(scores))
    if not noalloc:
        args += [_ptr(ws), ws.numel() * ws.element_size()]
    args.append(_stream(q))
    _check(fn(*args))
    return out, lse


def lvq_decode_attn(q, page_table, index_pages, bf16_pages, bf16_table, codebooks, t, pos,
                    seq_len, q_end, rope_tab, shp: AttnShape, out=None, lse=None, ws=None):
    """Decode attention at loop step t; returns (out [B][Hq][d] f32, lse [B][Hq] f32)."""
    return _attn_call(lib().lvq_decode_attn, q, page_table, index_pages, bf16_pages, bf16_table,
                      codebooks, t, pos, seq_len, q_end, rope_tab, shp, out, lse, ws)


def lvq_decode_attn_noalloc(q, page_table, index_pages, bf16_pages, bf16_table, codebooks, t, pos,
                            seq_len, q_end, rope_tab, shp: AttnShape, out, lse):
    """lvq_decode_attn without a workspace (the library's fixed scratch array): the caller
    passes the outputs, so the call allocates nothing.  Returns (out, lse)."""
    if out is None or lse is None:
        raise ValueError("lvq_decode_attn_noalloc needs the caller's out and lse tensors")
    return _attn_call(lib().lvq_decode_attn_noalloc, q, page_table, index_pages, bf16_pages, bf16_table,
                      codebooks, t, pos, seq_len, q_end, rope_tab, shp, out, lse, None, noalloc=True)


def lvq_decode_scores(q, page_table, index_pages, bf16_pages, bf16_table, codebooks, t, pos,
                      seq_len, q_end, rope_tab, shp: AttnShape, out=None, lse=None, ws=None, scores=None):
    """Test probe: (out, lse, scores [B][Hq][max_seq_len] f32).  Without a scores tensor
    one is allocated NaN-filled, so positions the call does not write stay NaN."""
    if scores is None:
        scores = torch.full((shp.B, shp.Hq, shp.max_seq_len), math.nan, dtype=torch.float32, device=q.device)
    out, lse = _attn_call(lib().lvq_decode_scores, q, page_table, index_pages, bf16_pages,
                          bf16_table, codebooks, t, pos, seq_len, q_end, rope_tab, shp, out, lse,
                          ws, scores=scores)
    return out, lse, scores


# ---------------------------------------------------------------- paged cache manager
CACHE_ERRORS = {1: "coded pool empty", 2: "bf16 pool empty", 4: "sequence beyond max_pages",
                8: "window beyond bf16_row"}


class PagedCache:
    """Device state of the paged cache manager (lvq_cache) in torch int32 tensors.

    The tensors page_table, bf16_table, seq_len and q_end are the ones lvq_decode_attn
    takes; re_src / re_dst feed lvq_reencode_pages between end_token and commit.  Every
    method only marshals arguments; the bookkeeping runs in the library's kernels.
    """

    def __init__(self, B: int, max_pages: int, n_sink: int, n_recent: int, n_index_pages: int,
                 n_bf16_pages: int, bf16_row: int | None = None, device="cuda"):
        if bf16_row is None:
            bf16_row = lib().lvq_cache_min_bf16_row(n_recent)
        i32 = dict(dtype=torch.int32, device=device)
        self.page_table = torch.empty((B, max_pages), **i32)
        self.bf16_table = torch.empty((B, bf16_row), **i32)
        self.seq_len = torch.empty(B, **i32)
        self.q_end = torch.empty(B, **i32)
        self.index_free = torch.empty(max(n_index_pages, 1), **i32)
        self.bf16_free = torch.empty(max(n_bf16_pages, 1), **i32)
        self.counters = torch.empty(4, **i32)
        self.re_src = torch.empty(B, **i32)
        self.re_dst = torch.empty(B, **i32)
        self.desc = CacheDesc(B, max_pages, bf16_row, n_sink, n_recent, n_index_pages, n_bf16_pages,
                              *[_ptr(t) for t in (self.page_table, self.bf16_table, self.seq_len, self.q_end,
                                                  self.index_free, self.bf16_free, self.counters,
                                                  self.re_src, self.re_dst)])
        self.B, self.max_pages, self.bf16_row = B, max_pages, bf16_row
        self.n_sink, self.n_recent = n_sink, n_recent
        self.n_index_pages, self.n_bf16_pages = n_index_pages, n_bf16_pages
        self.init()

    def _s(self):
        return _stream(self.seq_len)

    def init(self):
        _check(lib().lvq_cache_init(ctypes.byref(self.desc), self._s()))

    def prefill(self, lengths):
        _dev(lengths, "lengths", I32, 1)
        if lengths.numel() != self.B:
            raise ValueError("lengths must have B entries")
        _check(lib().lvq_cache_prefill(ctypes.byref(self.desc), _ptr(lengths), self._s()))

    def store_tokens(self, b: int, first: int, k, v, bf16_pages):
        """k, v bf16 [T][n][H][d]: tokens first .. first+n-1 of sequence b."""
        _dev(k, "k", BF16, 4)
        _dev(v, "v", BF16, 4)
        _dev(bf16_pages, "bf16_pages", BF16, 6)
        if k.shape != v.shape:
            raise ValueError("k and v differ in shape")
        T, n, H, d = k.shape
        self._check_pool(bf16_pages, T, H, d)
        _check(lib().lvq_cache_store_tokens(ctypes.byref(self.desc), b, first, n, _ptr(k), _ptr(v), T, H, d,
                                            _ptr(bf16_pages), self._s()))

    def begin_token(self):
        _check(lib().lvq_cache_begin_token(ctypes.byref(self.desc), self._s()))

    def append(self, t0: int, k, v, bf16_pages):
        """k, v bf16 [n_steps][B][H][d]: the new token at loop steps t0 .. t0+n_steps-1."""
        _dev(k, "k", BF16, 4)
        _dev(v, "v", BF16, 4)
        _dev(bf16_pages, "bf16_pages", BF16, 6)
        if k.shape != v.shape or k.shape[1] != self.B:
            raise ValueError("k and v must both be [n_steps][B][H][d]")
        n_steps, _, H, d = k.shape
        T = bf16_pages.shape[1]
        self._check_pool(bf16_pages, T, H, d)
        _check(lib().lvq_cache_append(ctypes.byref(self.desc), t0, n_steps, _ptr(k), _ptr(v), T, H, d,
                                      _ptr(bf16_pages), self._s()))

    def end_token(self):
        _check(lib().lvq_cache_end_token(ctypes.byref(self.desc), self._s()))

    def commit(self):
        _check(lib().lvq_cache_commit(ctypes.byref(self.desc), self._s()))

    def release(self, mask):
        _dev(mask, "mask", I32, 1)
        if mask.numel() != self.B:
            raise ValueError("mask must have B entries")
        _check(lib().lvq_cache_release(ctypes.byref(self.desc), _ptr(mask), self._s()))

    def errors(self) -> int:
        """Sticky error bits (synchronises with the device)."""
        return int(self.counters[2].item())

    def _check_pool(self, pool, T, H, d):
        if tuple(pool.shape[1:]) != (T, H, 2, PAGE, d) or pool.shape[0] != self.n_bf16_pages:
            raise ValueError(f"bf16_pages must be [{self.n_bf16_pages}][{T}][{H}][2][8][{d}]")


# ---------------------------------------------------------------- multi-row attention
def lvq_rows_attn_workspace_bytes(shp: RowsShape) -> int:
    return lib().lvq_rows_attn_workspace_bytes(ctypes.byref(shp))


def lvq_rows_attn(q, page_table, index_pages, bf16_pages, bf16_table, codebooks, t, pos, prefix_len,
                  q_end, rope_tab, shp: RowsShape, k_new=None, v_new=None, out=None, lse=None, ws=None):
    """Query rows q [B][NQ][Hq][d] over the paged prefix (and the chunk's own keys k_new/v_new
    [B][NQ][H][d], causally); returns (out [B][NQ][Hq][d] f32, lse [B][NQ][Hq] f32)."""
    _dev(q, "q", BF16, 4)
    for name, x in (("page_table", page_table), ("bf16_table", bf16_table)):
        _dev(x, name, I32, 2)
    _dev(index_pages, "index_pages", U8, 6)
    _dev(bf16_pages, "bf16_pages", BF16, 6)
    _dev(codebooks, "codebooks", BF16, 7)
    for name, x in (("pos", pos), ("prefix_len", prefix_len), ("q_end", q_end)):
        _dev(x, name, I32, 1)
    _dev(rope_tab, "rope_tab", F32, 1)
    if (k_new is None) != (v_new is None):
        raise ValueError("k_new and v_new go together")
    if k_new is not None:
        _dev(k_new, "k_new", BF16, 4)
        _dev(v_new, "v_new", BF16, 4)
    if tuple(q.shape) != (shp.B, shp.NQ, shp.Hq, shp.d):
        raise ValueError("q must be [B][NQ][Hq][d] of the shape")
    if k_new is not None:
        _expect(k_new, "k_new", (shp.B, shp.NQ, shp.H, shp.d))
        _expect(v_new, "v_new", (shp.B, shp.NQ, shp.H, shp.d))
    _expect(page_table, "page_table", (shp.B, shp.max_pages))
    _expect(bf16_table, "bf16_table", (shp.B, shp.bf16_row))
    for name, x in (("pos", pos), ("prefix_len", prefix_len), ("q_end", q_end)):
        _expect(x, name, (shp.B,))
    _expect(index_pages, "index_pages", _index_pool_shape(shp.n_index_pages, shp.T, shp.Tc, shp.G, shp.H, shp.d))
    _expect(bf16_pages, "bf16_pages", (shp.n_bf16_pages, shp.T, shp.H, 2, PAGE, shp.d))
    _expect(codebooks, "codebooks", _book_shape(shp.T, shp.Tc, shp.G, shp.H, shp.d))
    if rope_tab.numel() * 4 < lvq_rope_table_bytes(shp.rope_max_len, shp.d):
        raise ValueError("rope table too small")
    dev = q.device
    if out is None:
        out = torch.empty((shp.B, shp.NQ, shp.Hq, shp.d), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((shp.B, shp.NQ, shp.Hq), dtype=torch.float32, device=dev)
    _dev(out, "out", F32)
    _dev(lse, "lse", F32)
    _expect(out, "out", (shp.B, shp.NQ, shp.Hq, shp.d))
    _expect(lse, "lse", (shp.B, shp.NQ, shp.Hq))
    need = lvq_rows_attn_workspace_bytes(shp)
    if ws is None:
        ws = torch.empty(max(need, 4), dtype=torch.uint8, device=dev)
    _check(lib().lvq_rows_attn(_ptr(q), None if k_new is None else _ptr(k_new),
                               None if v_new is None else _ptr(v_new), _ptr(page_table), _ptr(index_pages),
                               _ptr(bf16_pages), _ptr(bf16_table), _ptr(codebooks), t, _ptr(pos),
                               _ptr(prefix_len), _ptr(q_end), _ptr(rope_tab), ctypes.byref(shp), _ptr(out),
                               _ptr(lse), _ptr(ws), ws.numel() * ws.element_size(), _stream(q)))
    return out, lse


def make_rows_shape(B, NQ, H, Hq, d, T, Tc, G, n_sink, max_pages, bf16_row, n_index_pages, n_bf16_pages,
                    max_prefix, rope_max_len, n_splits=0, scale=0.0, rejected=None) -> RowsShape:
    return RowsShape(B, NQ, H, Hq, d, T, Tc, G, n_sink, max_pages, bf16_row, n_index_pages, n_bf16_pages,
                     max_prefix, rope_max_len, n_splits, scale, _counter_ptr(rejected))
