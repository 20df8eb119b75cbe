"""Moves a test cache to the GPU and calls the library through its binding."""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

import sub_bit_loop_amd as lvq


@dataclass
class DevCache:
    host: object
    q: torch.Tensor
    page_table: torch.Tensor
    index_pages: torch.Tensor
    bf16_pages: torch.Tensor
    bf16_table: torch.Tensor
    codebooks: torch.Tensor
    pos: torch.Tensor
    seq_len: torch.Tensor
    q_end: torch.Tensor
    rope: torch.Tensor
    rope_max_len: int
    max_seq_len: int


def _t(x, dev, dtype=None):
    a = np.ascontiguousarray(x)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(dev)


def to_dev(cache, dev="cuda", max_seq_len: int | None = None, rope_base: float = 10000.0) -> DevCache:
    msl = int(max_seq_len or max(int(cache.seq_len.max()), 1))
    rml = int(max(msl, int(cache.pos.max()))) + 1
    pt = cache.page_table
    need = (msl + 7) // 8
    if pt.shape[1] < need:
        pt = np.concatenate([pt, np.full((pt.shape[0], need - pt.shape[1]), -1, np.int32)], 1)
    return DevCache(cache, _t(cache.q, dev), _t(pt, dev), _t(cache.index_pages, dev),
                    _t(cache.bf16_pages, dev), _t(cache.bf16_table, dev), _t(cache.codebooks, dev),
                    _t(cache.pos.astype(np.int32), dev), _t(cache.seq_len.astype(np.int32), dev),
                    _t(cache.q_end.astype(np.int32), dev),
                    lvq.lvq_rope_tables(rml, cache.d, rope_base, device=dev), rml, msl)


def shape_of(dc: DevCache, n_splits: int = 0, rejected=None, scale: float = 0.0) -> lvq.AttnShape:
    c = dc.host
    return lvq.make_shape(c.B, c.H, c.Hq, c.d, c.T, c.Tc, c.G, c.n_sink, dc.page_table.shape[1],
                          dc.bf16_table.shape[1], dc.index_pages.shape[0], dc.bf16_pages.shape[0],
                          dc.max_seq_len, dc.rope_max_len, n_splits, scale=scale, rejected=rejected)


def gpu_attn(dc: DevCache, t: int, n_splits: int = 0, scores: bool = False, q=None, rejected=None,
             scale: float = 0.0):
    shp = shape_of(dc, n_splits, rejected, scale)
    qq = dc.q[t] if q is None else q
    fn = lvq.lvq_decode_scores if scores else lvq.lvq_decode_attn
    res = fn(qq.contiguous(), dc.page_table, dc.index_pages, dc.bf16_pages, dc.bf16_table,
             dc.codebooks, t, dc.pos, dc.seq_len, dc.q_end, dc.rope, shp)
    torch.cuda.synchronize()
    return res


def attn_close(got, ref, atol=2e-3, rtol=1e-2, rel_floor=0.2):
    """The attention acceptance: max-abs <= atol over every element AND max-rel <= rtol
    over the elements with |ref| >= rel_floor (a relative error means nothing near zero).
    Returns (ok, max_abs, max_rel)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    big = np.abs(ref) >= rel_floor
    mabs = float(err.max()) if err.size else 0.0
    mrel = float((err[big] / np.abs(ref[big])).max()) if big.any() else 0.0
    ok = bool(np.isfinite(got).all()) and mabs <= atol and mrel <= rtol
    return ok, mabs, mrel
