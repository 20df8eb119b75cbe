"""Builds seeded LoopVQ caches for tests: synthetic tokens, fixture codebooks,
index pages encoded by the oracle (or drawn at random), bf16 pages, queries."""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

import synth
from oracle import lvq_oracle as orc


@dataclass
class Cache:
    B: int
    H: int
    Hq: int
    d: int
    T: int
    Tc: int
    G: int
    n_sink: int
    n_recent: int
    seq_len: np.ndarray
    q_end: np.ndarray
    pos: np.ndarray
    page_table: np.ndarray
    index_pages: np.ndarray
    bf16_pages: np.ndarray
    bf16_table: np.ndarray
    codebooks: np.ndarray
    q: np.ndarray                   # [T][B][Hq][d] bf16 bits
    k_tokens: list = field(default_factory=list)
    v_tokens: list = field(default_factory=list)

    @property
    def c(self):
        return self.G // self.Tc

    @property
    def ng(self):
        return self.d // self.c

    @property
    def nblk(self):
        return self.T // self.Tc

    def shape(self, rope_base=10000.0) -> orc.AttnShape:
        return orc.AttnShape(self.B, self.H, self.Hq, self.d, self.T, self.Tc, self.G,
                             self.n_sink, rope_base)

    def oracle_attn(self, t, **kw):
        return orc.decode_attn(self.shape(), self.q[t], self.page_table, self.index_pages,
                               self.bf16_pages, self.bf16_table, self.codebooks, t, self.pos,
                               self.seq_len, self.q_end, **kw)


def build_cache(config: int, B: int, lengths, H: int, d: int, T: int, Tc: int, G: int,
                n_sink: int, n_recent: int, Hq: int | None = None, books: str = "kmeans",
                index: str = "oracle", shuffle: bool = True, q_end=None,
                book_samples: int = 4096, keep_tokens: bool = True) -> Cache:
    Hq = H if Hq is None else Hq
    lengths = np.asarray(lengths, dtype=np.int32)
    rk = np.random.default_rng(synth.seed_for(config, synth.STREAM_K))
    rv = np.random.default_rng(synth.seed_for(config, synth.STREAM_V))
    sc_k = synth.channel_scales(rk, H, d)
    sc_v = synth.channel_scales(rv, H, d)
    ks, vs = [], []
    for b in range(B):
        ks.append(synth.f32_to_bf16_bits(synth.gen_kv(rk, T, int(lengths[b]), H, d, sc_k)))
        vs.append(synth.f32_to_bf16_bits(synth.gen_kv(rv, T, int(lengths[b]), H, d, sc_v)))
    if q_end is None:
        q_end = np.array([synth.prefill_q_end(int(L), n_recent) for L in lengths], dtype=np.int32)
    q_end = np.asarray(q_end, dtype=np.int32)
    if books == "kmeans":
        cb = synth.kmeans_codebooks(config, T, Tc, G, H, d, sc_k, sc_v, n_samples=book_samples)
    else:
        cb = synth.random_codebooks(np.random.default_rng(synth.seed_for(config, synth.STREAM_BOOKS)),
                                    T, Tc, G, H, d, scale=2.0)
    c = G // Tc
    ng, nblk = d // c, T // Tc
    n_pages = [int(qe) // 8 for qe in q_end]
    max_pages = max(1, max((int(L) + 7) // 8 for L in lengths))
    rp = np.random.default_rng(synth.seed_for(config, synth.STREAM_PAGES))
    if shuffle:
        pt, pool = synth.shuffled_page_table(rp, n_pages, max_pages)
    else:
        pt = np.full((B, max_pages), -1, dtype=np.int32)
        o = 0
        for b, n in enumerate(n_pages):
            pt[b, :n] = np.arange(o, o + n)
            o += n
        pool = o
    pool = max(pool, 1)
    if index == "oracle":
        ip = np.zeros((pool, nblk, H, 2, 8, ng), dtype=np.uint8)
        for b in range(B):
            qe = int(q_end[b])
            if qe == 0:
                continue
            for kv, toks in ((0, ks[b]), (1, vs[b])):
                r = orc.encode(toks[:, :qe], cb, kv, T, Tc, G)
                orc.scatter_index_pages(r.idx, kv, pt[b, :qe // 8], ip)
    else:
        ip = synth.random_index_pages(rp, pool, nblk, H, ng)
    bp, lay = synth.pack_bf16_pages(ks, vs, q_end, T, H, d, rng=rp if shuffle else None)
    rq = np.random.default_rng(synth.seed_for(config, synth.STREAM_Q))
    q = synth.gen_queries(rq, T, B, Hq, d)
    return Cache(B, H, Hq, d, T, Tc, G, n_sink, n_recent, lengths.copy(), q_end,
                 lengths.copy(), pt, ip, bp, lay.bf16_table, cb, q,
                 ks if keep_tokens else [], vs if keep_tokens else [])


def build_cache_light(config: int, B: int, lengths, H: int, d: int, T: int, Tc: int, G: int,
                      n_sink: int, n_recent: int, Hq: int | None = None, books: str = "random",
                      book_samples: int = 1024) -> Cache:
    """Full-size cache without generating every token: coded pages hold uniform random
    indices; only the bf16 parts (page 0 and the recent window) are drawn from the
    generator.  For attention tests at real context lengths."""
    import torch
    Hq = H if Hq is None else Hq
    lengths = np.asarray(lengths, dtype=np.int32)
    rk = np.random.default_rng(synth.seed_for(config, synth.STREAM_K))
    rv = np.random.default_rng(synth.seed_for(config, synth.STREAM_V))
    sc_k = synth.channel_scales(rk, H, d)
    sc_v = synth.channel_scales(rv, H, d)
    q_end = np.array([synth.prefill_q_end(int(L), n_recent) for L in lengths], dtype=np.int32)
    c = G // Tc
    ng, nblk = d // c, T // Tc
    if books == "kmeans":
        torch.set_num_threads(min(16, torch.get_num_threads()))
        rb = np.random.default_rng(synth.seed_for(config, synth.STREAM_BOOKS))
        sk = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(synth.gen_kv(rb, T, book_samples, H, d, sc_k)))
        sv = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(synth.gen_kv(rb, T, book_samples, H, d, sc_v)))
        kw = dict(device="cpu", dtype=torch.float32)
        cb = np.stack([synth.codebooks_from_samples(sk, Tc, G, config * 7 + 1, **kw),
                       synth.codebooks_from_samples(sv, Tc, G, config * 7 + 2, **kw)], axis=1)
    else:
        rb = np.random.default_rng(synth.seed_for(config, synth.STREAM_BOOKS))
        cb = np.ascontiguousarray(synth.random_codebooks(rb, T, Tc, G, H, d, scale=1.0))
        # put the books on the data's per-channel scale
        f = synth.bf16_bits_to_f32(cb).astype(np.float32)
        for kv, sc in ((0, sc_k), (1, sc_v)):
            scl = sc.reshape(H, ng, c)                    # [H][ng][c]
            f[:, kv] *= scl[None, :, :, None, None, :]
        cb = synth.f32_to_bf16_bits(f)
    n_pages = [int(qe) // 8 for qe in q_end]
    max_pages = max(1, max((int(L) + 7) // 8 for L in lengths))
    rp = np.random.default_rng(synth.seed_for(config, synth.STREAM_PAGES))
    pt, pool = synth.shuffled_page_table(rp, n_pages, max_pages)
    ip = synth.random_index_pages(rp, max(pool, 1), nblk, H, ng)
    fk, fv, rk_, rv_ = [], [], [], []
    for b in range(B):
        L = int(lengths[b])
        base = (int(q_end[b]) // 8) * 8
        fk.append(synth.f32_to_bf16_bits(synth.gen_kv(rk, T, min(8, L), H, d, sc_k)))
        fv.append(synth.f32_to_bf16_bits(synth.gen_kv(rv, T, min(8, L), H, d, sc_v)))
        rk_.append(synth.f32_to_bf16_bits(synth.gen_kv(rk, T, L - base, H, d, sc_k)))
        rv_.append(synth.f32_to_bf16_bits(synth.gen_kv(rv, T, L - base, H, d, sc_v)))
        if base == 0:   # page 0 is also a recent page: keep both copies identical
            n = min(8, L)
            rk_[-1][:, :n] = fk[-1][:, :n]
            rv_[-1][:, :n] = fv[-1][:, :n]
    bp, lay = synth.pack_bf16_pages_parts(fk, fv, rk_, rv_, q_end, lengths, T, H, d, rng=rp)
    rq = np.random.default_rng(synth.seed_for(config, synth.STREAM_Q))
    q = synth.gen_queries(rq, T, B, Hq, d)
    return Cache(B, H, Hq, d, T, Tc, G, n_sink, n_recent, lengths.copy(), q_end, lengths.copy(),
                 pt, ip, bp, lay.bf16_table, cb, q)


def build_cache_generated(config: int, B: int, lengths, H: int, d: int, T: int, Tc: int, G: int,
                          n_sink: int, n_recent: int, book_samples: int = 4096) -> Cache:
    """Full-size cache from the generator's own tokens, built with torch on the GPU (input
    preparation only, none of the library's kernels): AR(1) keys and values per sequence,
    k-means++ / 10-Lloyd codebooks fitted on `book_samples` seeded samples, and every coded
    token's index the nearest codeword by torch's float32 distance matmul and argmin.  The
    indices are therefore realistic codes (not uniform draws); where float32 rounding picks
    a near-tied neighbour the cache is still a valid input, since attention parity reads the
    same pages on both sides."""
    import torch
    dev = torch.device("cuda")
    lengths = np.asarray(lengths, dtype=np.int32)
    rk = np.random.default_rng(synth.seed_for(config, synth.STREAM_K))
    rv = np.random.default_rng(synth.seed_for(config, synth.STREAM_V))
    sc_k = synth.channel_scales(rk, H, d)
    sc_v = synth.channel_scales(rv, H, d)
    c = G // Tc
    ng, nblk = d // c, T // Tc
    rb = np.random.default_rng(synth.seed_for(config, synth.STREAM_BOOKS))
    books = []
    for kv, sc in ((0, sc_k), (1, sc_v)):
        s = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(synth.gen_kv(rb, T, book_samples, H, d, sc)))
        books.append(synth.codebooks_from_samples(s, Tc, G, config * 7 + 1 + kv, device="cuda",
                                                  dtype=torch.float32))
    cb = np.ascontiguousarray(np.stack(books, axis=1))                 # [nblk][2][H][ng][Tc][256][c]
    cbf = torch.from_numpy(synth.bf16_bits_to_f32(cb).astype(np.float32)).to(dev)
    # joint codewords [nblk][2][H][ng][256][G], step-major inside the joint vector
    Cj = cbf.permute(0, 1, 2, 3, 5, 4, 6).reshape(nblk, 2, H, ng, 256, G).contiguous()
    cn = (Cj * Cj).sum(-1)                                              # [nblk][2][H][ng][256]
    q_end = np.array([synth.prefill_q_end(int(L), n_recent) for L in lengths], dtype=np.int32)
    n_pages = [int(qe) // 8 for qe in q_end]
    max_pages = max(1, max((int(L) + 7) // 8 for L in lengths))
    rp = np.random.default_rng(synth.seed_for(config, synth.STREAM_PAGES))
    pt, pool = synth.shuffled_page_table(rp, n_pages, max_pages)
    ip = np.zeros((max(pool, 1), nblk, H, 2, 8, ng), dtype=np.uint8)
    gen = torch.Generator(device=dev)
    fk, fv, rk_, rv_ = [], [], [], []
    for b in range(B):
        L, qe = int(lengths[b]), int(q_end[b])
        base = (qe // 8) * 8
        for kv, sc, first, rec in ((0, sc_k, fk, rk_), (1, sc_v, fv, rv_)):
            gen.manual_seed(synth.seed_for(config, kv) * 1009 + b)
            x = synth.gen_kv_torch(gen, T, L, H, d, sc, device=dev)     # bf16 [T][L][H][d]
            first.append(x[:, :min(8, L)].view(torch.int16).cpu().numpy().view(np.uint16))
            rec.append(x[:, base:L].view(torch.int16).cpu().numpy().view(np.uint16))
            if qe == 0:
                continue
            xf = x[:, :qe].float().reshape(nblk, Tc, qe, H, ng, c)
            J = xf.permute(0, 3, 4, 2, 1, 5).reshape(nblk, H, ng, qe, G)   # [nblk][H][ng][qe][G]
            idx = torch.empty((nblk, H, ng, qe), dtype=torch.uint8, device=dev)
            for beta in range(nblk):
                for h in range(H):
                    A = J[beta, h].contiguous()                          # [ng][qe][G]
                    Ct = Cj[beta, kv, h].transpose(1, 2).contiguous()    # [ng][G][256]
                    dist = cn[beta, kv, h][:, None, :] - 2.0 * torch.bmm(A, Ct)
                    idx[beta, h] = dist.argmin(-1).to(torch.uint8)
            idx = idx.view(nblk, H, ng, qe // 8, 8).permute(3, 0, 1, 4, 2).cpu().numpy()  # [pg][nblk][H][8][ng]
            ip[pt[b, :qe // 8], :, :, kv] = idx
            del x, xf, J, idx
    torch.cuda.empty_cache()
    bp, lay = synth.pack_bf16_pages_parts(fk, fv, rk_, rv_, q_end, lengths, T, H, d, rng=rp)
    rq = np.random.default_rng(synth.seed_for(config, synth.STREAM_Q))
    q = synth.gen_queries(rq, T, B, H, d)
    return Cache(B, H, H, d, T, Tc, G, n_sink, n_recent, lengths.copy(), q_end, lengths.copy(),
                 pt, ip, bp, lay.bf16_table, cb, q)
