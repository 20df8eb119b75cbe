"""Seeded generators for LoopVQ-shaped synthetic workloads.

The recipe stands in for keys/values of a looped transformer (Ouro-style),
whose real activations are not available:

* Per (layer, head, token) latent that is AR(1) across loop steps.  The
  adjacent-step correlation rises linearly from 0.69 (first pair of steps) to
  0.94 (last pair), the loop-axis redundancy figures of the LoopVQ summary
  (onedev.kr/papers/1681, section "어떻게 동작하나"; rit.work LoopVQ article,
  section "Общие веса не сокращают память контекста").
* Cross-channel correlation about 0.16 inside a step: the innovation is
  ``0.4 * s + sqrt(0.84) * e`` with ``s`` one shared N(0,1) scalar per
  (token, head, step) and ``e`` iid per channel, so corr = 0.4**2 = 0.16.
* Per (head, channel) scale drawn lognormal(0, 0.5) and two seeded outlier
  channels per head multiplied by 8.
* Tokens iid, generated in float32 and rounded to bfloat16 (round to nearest
  even).  Keys are pre-RoPE.  Values are an independent draw.
* Queries N(0, 1) per channel, bfloat16, one per loop step.
* Codebook fixture: k-means++ seeding and 10 Lloyd iterations on 4096 seeded
  joint-vector samples per codebook, rounded to bfloat16.  This is input
  preparation (the method's calibration step is out of the hot path); its
  quality is never graded.

Everything is keyed by ``seed_for(config, stream)`` so a run is reproducible.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

__all__ = [
    "STREAM_K", "STREAM_V", "STREAM_Q", "STREAM_BOOKS", "STREAM_PAGES",
    "STREAM_LENGTHS", "STREAM_NEEDLE", "seed_for", "f32_to_bf16_bits",
    "bf16_bits_to_f32", "loop_rhos", "channel_scales", "gen_kv", "gen_queries",
    "kmeans_codebooks", "codebooks_from_samples", "shuffled_page_table",
    "uniform_lengths", "random_index_pages", "random_codebooks",
    "CacheLayout", "pack_bf16_pages", "pack_bf16_pages_parts", "prefill_q_end",
    "gen_kv_torch", "gen_queries_torch",
]

STREAM_K, STREAM_V, STREAM_Q, STREAM_BOOKS, STREAM_PAGES, STREAM_LENGTHS, STREAM_NEEDLE = range(7)

PAGE = 8        # tokens per cache page
NCODES = 256    # codewords per codebook (8-bit index)


def seed_for(config: int, stream: int) -> int:
    """Seed of one random stream of one workload configuration."""
    return 1000 * int(config) + int(stream)


# ----------------------------------------------------------------------------
# bfloat16 bit patterns
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    r[np.isnan(x)] = 0x7FC0
    return r


def bf16_bits_to_f32(u) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact)."""
    u = np.ascontiguousarray(np.asarray(u, dtype=np.uint16))
    return (u.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------
# keys / values / queries
# ----------------------------------------------------------------------------
def loop_rhos(T: int) -> np.ndarray:
    """AR(1) coefficient between step t-1 and t, for t = 1..T-1 (linear 0.69 -> 0.94)."""
    if T <= 1:
        return np.zeros(0)
    return np.linspace(0.69, 0.94, T - 1)


def channel_scales(rng: np.random.Generator, H: int, d: int, n_outliers: int = 2,
                   outlier_gain: float = 8.0) -> np.ndarray:
    """Per (head, channel) scale: lognormal(0, 0.5) with ``n_outliers`` channels x8 per head."""
    s = rng.lognormal(mean=0.0, sigma=0.5, size=(H, d))
    for h in range(H):
        ch = rng.choice(d, size=min(n_outliers, d), replace=False)
        s[h, ch] *= outlier_gain
    return s


def gen_kv(rng: np.random.Generator, T: int, N: int, H: int, d: int,
           scales: np.ndarray, dtype=np.float32) -> np.ndarray:
    """Loop-correlated tokens, float ``[T][N][H][d]`` (not yet rounded to bf16)."""
    rhos = loop_rhos(T)
    out = np.empty((T, N, H, d), dtype=dtype)
    c_shared, c_own = 0.4, math.sqrt(0.84)
    z = None
    for t in range(T):
        s = rng.standard_normal((N, H, 1))
        e = rng.standard_normal((N, H, d))
        eps = c_shared * s + c_own * e
        if t == 0:
            z = eps
        else:
            r = rhos[t - 1]
            z = r * z + math.sqrt(1.0 - r * r) * eps
        out[t] = (z * scales[None, :, :]).astype(dtype)
    return out


def gen_queries(rng: np.random.Generator, T: int, B: int, Hq: int, d: int) -> np.ndarray:
    """bf16 bit patterns ``[T][B][Hq][d]``: one query per loop step, N(0,1) per channel."""
    return f32_to_bf16_bits(rng.standard_normal((T, B, Hq, d)).astype(np.float32))


# ----------------------------------------------------------------------------
# codebook fixtures
# ----------------------------------------------------------------------------
def _kmeans_batched(X, K: int, iters: int, gen):
    """k-means++ seeding + Lloyd iterations on a batch of independent problems.

    X: torch tensor (nb, S, G).  Empty clusters keep their previous centroid.
    """
    import torch
    nb, S, G = X.shape
    dev = X.device
    ar = torch.arange(nb, device=dev)
    C = torch.empty((nb, K, G), dtype=X.dtype, device=dev)
    first = torch.randint(S, (nb,), generator=gen, device=dev)
    C[:, 0] = X[ar, first]
    d2 = ((X - C[:, 0:1]) ** 2).sum(-1)
    for k in range(1, K):
        tot = d2.sum(-1, keepdim=True)
        p = torch.where(tot > 0, d2 / tot.clamp_min(1e-300), torch.full_like(d2, 1.0 / S))
        cdf = p.cumsum(-1)
        u = torch.rand((nb, 1), generator=gen, device=dev, dtype=X.dtype) * cdf[:, -1:]
        idx = torch.searchsorted(cdf, u).clamp_max(S - 1).squeeze(-1)
        C[:, k] = X[ar, idx]
        d2 = torch.minimum(d2, ((X - C[:, k:k + 1]) ** 2).sum(-1))
    xx = (X * X).sum(-1, keepdim=True)
    ones = torch.ones((nb, S), dtype=X.dtype, device=dev)
    for _ in range(iters):
        dist = xx - 2.0 * torch.bmm(X, C.transpose(1, 2).contiguous()) + (C * C).sum(-1)[:, None, :]
        a = dist.argmin(-1)
        sums = torch.zeros((nb, K, G), dtype=X.dtype, device=dev)
        sums.scatter_add_(1, a[..., None].expand(-1, -1, G), X)
        cnt = torch.zeros((nb, K), dtype=X.dtype, device=dev)
        cnt.scatter_add_(1, a, ones)
        newC = sums / cnt.clamp_min(1.0)[..., None]
        C = torch.where(cnt[..., None] > 0, newC, C)
    return C


def codebooks_from_samples(samples: np.ndarray, Tc: int, G: int, seed: int, K: int = NCODES,
                           iters: int = 10, device: str = "cpu", dtype=None) -> np.ndarray:
    """bf16 codebooks ``[nblk][H][ng][Tc][K][c]`` fitted to tokens ``samples[T][S][H][d]``.

    The fixture must be emitted in the cache's codebook layout, so it arranges
    its training samples the same way: block ``b`` of ``Tc`` steps, group ``g``
    of ``c = G / Tc`` contiguous channels, step-major inside the G-vector.
    """
    import torch
    T, S, H, d = samples.shape
    c = G // Tc
    nblk, ng = T // Tc, d // c
    X = np.asarray(samples, dtype=np.float64)
    X = X.reshape(nblk, Tc, S, H, ng, c).transpose(0, 3, 4, 2, 1, 5).reshape(nblk * H * ng, S, G)
    if dtype is None:
        dtype = torch.float64 if device == "cpu" else torch.float32
    Xt = torch.from_numpy(np.ascontiguousarray(X)).to(device=device, dtype=dtype)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    C = _kmeans_batched(Xt, K, iters, gen).to("cpu", torch.float64).numpy()
    C = C.reshape(nblk, H, ng, K, Tc, c).transpose(0, 1, 2, 4, 3, 5)
    return f32_to_bf16_bits(C.astype(np.float32))


def kmeans_codebooks(config: int, T: int, Tc: int, G: int, H: int, d: int,
                     scales_k: np.ndarray, scales_v: np.ndarray, n_samples: int = 4096,
                     device: str = "cpu") -> np.ndarray:
    """Codebooks ``[nblk][2][H][ng][Tc][256][c]`` (bf16 bits) for keys (0) and values (1)."""
    rng = np.random.default_rng(seed_for(config, STREAM_BOOKS))
    sk = gen_kv(rng, T, n_samples, H, d, scales_k)
    sv = gen_kv(rng, T, n_samples, H, d, scales_v)
    # the samples go through the same bf16 rounding as the cache contents
    sk = bf16_bits_to_f32(f32_to_bf16_bits(sk))
    sv = bf16_bits_to_f32(f32_to_bf16_bits(sv))
    bk = codebooks_from_samples(sk, Tc, G, seed_for(config, STREAM_BOOKS) * 7 + 1, device=device)
    bv = codebooks_from_samples(sv, Tc, G, seed_for(config, STREAM_BOOKS) * 7 + 2, device=device)
    return np.ascontiguousarray(np.stack([bk, bv], axis=1))


def random_codebooks(rng: np.random.Generator, T: int, Tc: int, G: int, H: int, d: int,
                     scale: float = 1.0) -> np.ndarray:
    """Gaussian codebooks ``[nblk][2][H][ng][Tc][256][c]`` (bf16 bits), for layout/timing cases."""
    c = G // Tc
    shape = (T // Tc, 2, H, d // c, Tc, NCODES, c)
    return f32_to_bf16_bits((scale * rng.standard_normal(shape)).astype(np.float32))


# ----------------------------------------------------------------------------
# cache bookkeeping inputs
# ----------------------------------------------------------------------------
def shuffled_page_table(rng: np.random.Generator, n_pages: list, max_pages: int,
                        pool: int | None = None) -> tuple[np.ndarray, int]:
    """Page table ``[B][max_pages]`` (int32, -1 padded) over a shuffled pool.

    Sequence ``b`` owns ``n_pages[b]`` logical pages; their physical ids are a
    seeded random permutation of ``range(pool)``.  Returns (table, pool).
    """
    total = int(sum(n_pages))
    pool = total if pool is None else int(pool)
    assert pool >= total
    perm = rng.permutation(pool).astype(np.int32)
    tab = np.full((len(n_pages), max_pages), -1, dtype=np.int32)
    o = 0
    for b, n in enumerate(n_pages):
        tab[b, :n] = perm[o:o + n]
        o += n
    return tab, pool


def uniform_lengths(rng: np.random.Generator, B: int, lo: int, hi: int) -> np.ndarray:
    """Sequence lengths uniform on [lo, hi] (inclusive), int32."""
    return rng.integers(lo, hi + 1, size=B).astype(np.int32)


def random_index_pages(rng: np.random.Generator, P: int, nblk: int, H: int, ng: int) -> np.ndarray:
    """Uniform uint8 code indices in the coded-page layout ``[P][nblk][H][2][8][ng]``."""
    return rng.integers(0, NCODES, size=(P, nblk, H, 2, PAGE, ng), dtype=np.uint8)


def prefill_q_end(L: int, n_recent: int) -> int:
    """End of the coded region right after prefill: 8 * floor((L - n_recent) / 8), clamped at 0."""
    return max(0, PAGE * ((L - n_recent) // PAGE))


@dataclass
class CacheLayout:
    """Where each sequence's bf16 pages live (sink copy of page 0 + recent pages)."""
    bf16_table: np.ndarray     # [B][1 + max_recent_pages] int32, -1 padded
    n_bf16_pages: int          # pool size


def pack_bf16_pages(k_tokens: list, v_tokens: list, q_end: np.ndarray, T: int, H: int, d: int,
                    rng: np.random.Generator | None = None, max_recent_pages: int | None = None):
    """Build the bf16 page pool ``[P'][T][H][2][8][d]`` (bf16 bits) and its table.

    ``k_tokens[b]`` / ``v_tokens[b]`` are bf16 bit arrays ``[T][L_b][H][d]`` of
    sequence ``b``.  Entry 0 of a table row is a copy of logical page 0 (the
    sink tokens live there); entries 1.. are the recent pages in logical order
    starting at logical page ``q_end[b] / 8``.  Unused slots of the last
    recent page are zero.  With ``rng`` the pool is shuffled.
    """
    first_k, first_v, rec_k, rec_v, lens = [], [], [], [], []
    for b in range(len(k_tokens)):
        L = k_tokens[b].shape[1]
        lo = (int(q_end[b]) // PAGE) * PAGE
        first_k.append(k_tokens[b][:, :PAGE])
        first_v.append(v_tokens[b][:, :PAGE])
        rec_k.append(k_tokens[b][:, lo:L])
        rec_v.append(v_tokens[b][:, lo:L])
        lens.append(L)
    return pack_bf16_pages_parts(first_k, first_v, rec_k, rec_v, q_end, lens, T, H, d, rng,
                                 max_recent_pages)


def pack_bf16_pages_parts(first_k, first_v, rec_k, rec_v, q_end, seq_len, T: int, H: int, d: int,
                          rng: np.random.Generator | None = None,
                          max_recent_pages: int | None = None):
    """As ``pack_bf16_pages`` from the parts that stay bf16: ``first_*[b]`` holds
    tokens 0..7 (``[T][<=8][H][d]``) and ``rec_*[b]`` tokens ``8*(q_end/8) .. L-1``."""
    B = len(first_k)
    rows = []
    for b in range(B):
        L = int(seq_len[b])
        first = int(q_end[b]) // PAGE
        last = (L + PAGE - 1) // PAGE
        rows.append([0] + list(range(first, last)))
    width = max(len(r) for r in rows) if max_recent_pages is None else 1 + max_recent_pages
    total = sum(len(r) for r in rows)
    perm = rng.permutation(total) if rng is not None else np.arange(total)
    pool = np.zeros((total, T, H, 2, PAGE, d), dtype=np.uint16)
    tab = np.full((B, width), -1, dtype=np.int32)
    o = 0
    for b in range(B):
        L = int(seq_len[b])
        base = (int(q_end[b]) // PAGE) * PAGE
        for j, lp in enumerate(rows[b]):
            pid = int(perm[o])
            o += 1
            tab[b, j] = pid
            lo, hi = lp * PAGE, min(L, lp * PAGE + PAGE)
            n = hi - lo
            if j == 0:
                src_k, src_v, off = first_k[b], first_v[b], 0
            else:
                src_k, src_v, off = rec_k[b], rec_v[b], lo - base
            pool[pid, :, :, 0, :n, :] = src_k[:, off:off + n].transpose(0, 2, 1, 3)
            pool[pid, :, :, 1, :n, :] = src_v[:, off:off + n].transpose(0, 2, 1, 3)
    return pool, CacheLayout(bf16_table=tab, n_bf16_pages=total)


# ----------------------------------------------------------------------------
# device-side variants of the same recipe (benchmark-scale inputs)
# ----------------------------------------------------------------------------
def gen_kv_torch(gen, T: int, N: int, H: int, d: int, scales, device="cuda"):
    """``gen_kv`` on a torch device: bf16 tensor ``[T][N][H][d]`` (same recipe, torch RNG)."""
    import torch
    rhos = loop_rhos(T)
    sc = torch.as_tensor(scales, dtype=torch.float32, device=device)
    out = torch.empty((T, N, H, d), dtype=torch.bfloat16, device=device)
    z = None
    for t in range(T):
        s = torch.randn((N, H, 1), generator=gen, device=device)
        e = torch.randn((N, H, d), generator=gen, device=device)
        eps = 0.4 * s + math.sqrt(0.84) * e
        if t == 0:
            z = eps
        else:
            r = float(rhos[t - 1])
            z = r * z + math.sqrt(1.0 - r * r) * eps
        out[t] = (z * sc[None]).to(torch.bfloat16)
    return out


def gen_queries_torch(gen, B: int, Hq: int, d: int, device="cuda"):
    """One bf16 query tensor ``[B][Hq][d]``, N(0,1) per channel, on a torch device."""
    import torch
    return torch.randn((B, Hq, d), generator=gen, device=device).to(torch.bfloat16)
