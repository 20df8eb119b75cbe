"""LoopVQ hot-path oracle: plain, slow, float64 CPU reference.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import or run this module; the product path
never does (it has no CPU fallback).  It shares no code with the HIP library:
layouts are re-implemented here from their documented definitions.

What it computes (all citations are to the LoopVQ pages):

* Joint loop-axis code (LoopVQ summary, onedev.kr/papers/1681, section
  "무엇과 다른가"; rit.work article, section "Один код описывает несколько
  шагов цикла"): the T loop steps are cut into contiguous blocks of Tc steps;
  one code covers c = G / Tc channels of every step of a block, so a code is
  the index of the codeword nearest to a G-dimensional joint vector, and each
  step keeps only its own c-channel share of that codeword.  With K = 256 the
  index is one byte, i.e. 8 / G bits per element whatever Tc is.
* Nearest codeword = smallest squared Euclidean distance (the summary, section
  "전제와 한계", computes the codebook distances with a matrix product, which
  is the expansion of the squared L2 norm); ties go to the lowest index.
* Pre-RoPE keys; RoPE applied to the reconstructed key inside attention
  (summary, section "무엇과 다른가").
* 8-token pages, bf16 sink and recent tokens, the rest stored as one index row
  per loop block; decode attention reads only the loop-step-t slice of each
  codeword and merges Flash-Decoding splits with a log-sum-exp (summary,
  section "전제와 한계"); values are reconstructed from codebooks as well and
  the coded part is merged with the uncompressed part (rit.work article,
  section "Когда LoopVQ меняет план развёртывания").

Readings where the pages are silent (rotate-half RoPE pairs (j, j + d/2) with
base 10000, softmax scale 1/sqrt(d), step-major element order inside the joint
vector, contiguous channel groups, one codebook per (loop block, K/V, head,
group), sink tokens taken from the retained bf16 copy of page 0) are the plain
readings; each is listed with its reason in the design notes.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

PAGE = 8
NCODES = 256
NEAR_TIE_REL = 1e-5


# ----------------------------------------------------------------------------
# inputs
# ----------------------------------------------------------------------------
def bf16_to_f64(u) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exact."""
    u = np.ascontiguousarray(np.asarray(u, dtype=np.uint16))
    return (u.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def check_divisibility(T: int, Tc: int, G: int, d: int) -> None:
    """Tc must divide T and G (summary, section "무엇과 다른가"); the c-channel groups must tile d."""
    if Tc <= 0 or T % Tc or G % Tc:
        raise ValueError(f"Tc={Tc} must divide T={T} and G={G}")
    c = G // Tc
    if d % c:
        raise ValueError(f"c=G/Tc={c} must divide d={d}")


# ----------------------------------------------------------------------------
# encoder
# ----------------------------------------------------------------------------
def joint_vectors(X: np.ndarray, Tc: int, G: int) -> np.ndarray:
    """Joint vectors ``x[beta][n][h][g][tau*c + i] = X[beta*Tc + tau][n][h][g*c + i]``.

    X: float ``[T][N][H][d]`` (one of K or V).  One joint vector gathers the
    same c channels of the Tc consecutive loop steps of a block (summary,
    section "무엇과 다른가"), step-major.
    """
    T, N, H, d = X.shape
    check_divisibility(T, Tc, G, d)
    c = G // Tc
    nblk, ng = T // Tc, d // c
    out = np.empty((nblk, N, H, ng, G), dtype=np.float64)
    for beta in range(nblk):
        for tau in range(Tc):
            step = X[beta * Tc + tau]
            for g in range(ng):
                out[beta, :, :, g, tau * c:(tau + 1) * c] = step[:, :, g * c:(g + 1) * c]
    return out


def joint_codewords(cb_half: np.ndarray) -> np.ndarray:
    """Codeword k of book (beta, h, g) as a G-vector: ``C[e = tau*c + i] = cb[beta][h][g][tau][k][i]``.

    cb_half: float ``[nblk][H][ng][Tc][256][c]`` (the K or the V half of the books).
    """
    nblk, H, ng, Tc, K, c = cb_half.shape
    out = np.empty((nblk, H, ng, K, Tc * c), dtype=np.float64)
    for tau in range(Tc):
        out[..., tau * c:(tau + 1) * c] = cb_half[:, :, :, tau, :, :]
    return out


@dataclass
class NearestResult:
    idx: np.ndarray        # chosen index, lowest among exact minima
    d1: np.ndarray         # best squared distance
    d2: np.ndarray         # second best squared distance (any other index)
    n_near: np.ndarray     # size of the near-tie set N(x)


def nearest_codeword(x: np.ndarray, C: np.ndarray, chunk: int = 1024) -> NearestResult:
    """Brute-force nearest codeword by squared L2, direct-difference form, float64.

    x: ``[n][G]``, C: ``[K][G]``.  D_k = sum_e (x_e - C_k[e])^2; the answer is the
    lowest k attaining the minimum.  The near-tie set is
    N(x) = {k : D_k - D_min <= 1e-5 * D_min} (the exact-zero set when D_min = 0).
    """
    n = x.shape[0]
    idx = np.empty(n, dtype=np.int64)
    d1 = np.empty(n)
    d2 = np.empty(n)
    nn = np.empty(n, dtype=np.int64)
    for s in range(0, n, chunk):
        xs = x[s:s + chunk]
        D = ((xs[:, None, :] - C[None, :, :]) ** 2).sum(-1)
        k = np.argmin(D, axis=1)            # first occurrence = lowest index
        best = D[np.arange(len(xs)), k]
        D2 = D.copy()
        D2[np.arange(len(xs)), k] = np.inf
        idx[s:s + chunk] = k
        d1[s:s + chunk] = best
        d2[s:s + chunk] = D2.min(axis=1)
        nn[s:s + chunk] = (D - best[:, None] <= NEAR_TIE_REL * best[:, None]).sum(axis=1)
    return NearestResult(idx, d1, d2, nn)


@dataclass
class EncodeResult:
    idx: np.ndarray        # uint8 [nblk][N][H][ng]
    d1: np.ndarray         # float64 [nblk][N][H][ng]
    d2: np.ndarray
    n_near: np.ndarray     # int  [nblk][N][H][ng]; > 1 marks a near tie


def encode(kv_bits: np.ndarray, codebooks_bits: np.ndarray, kv_sel: int, T: int, Tc: int,
           G: int) -> EncodeResult:
    """Encode one of K (kv_sel=0) / V (kv_sel=1): ``kv[T][N][H][d]`` -> ``idx[nblk][N][H][ng]``.

    codebooks_bits: bf16 ``[nblk][2][H][ng][Tc][256][c]``.  Encoding needs all Tc
    steps of a block to be present (summary, section "전제와 한계").
    """
    X = bf16_to_f64(kv_bits)
    T_, N, H, d = X.shape
    assert T_ == T
    J = joint_vectors(X, Tc, G)
    C = joint_codewords(bf16_to_f64(codebooks_bits)[:, kv_sel])
    nblk, ng = J.shape[0], J.shape[3]
    idx = np.empty((nblk, N, H, ng), dtype=np.uint8)
    d1 = np.empty((nblk, N, H, ng))
    d2 = np.empty((nblk, N, H, ng))
    nn = np.empty((nblk, N, H, ng), dtype=np.int64)
    for beta in range(nblk):
        for h in range(H):
            for g in range(ng):
                r = nearest_codeword(J[beta, :, h, g], C[beta, h, g])
                idx[beta, :, h, g] = r.idx
                d1[beta, :, h, g] = r.d1
                d2[beta, :, h, g] = r.d2
                nn[beta, :, h, g] = r.n_near
    return EncodeResult(idx, d1, d2, nn)


def scatter_index_pages(idx: np.ndarray, kv_sel: int, chunk_page: np.ndarray,
                        index_pages: np.ndarray) -> None:
    """Write dense rows ``idx[nblk][N][H][ng]`` into ``index_pages[P][nblk][H][2][8][ng]``.

    Token n goes to page ``chunk_page[n // 8]``, slot ``n % 8``, half ``kv_sel``:
    one index row per loop block in every coded page (summary, section "전제와 한계").
    """
    nblk, N, H, ng = idx.shape
    for n in range(N):
        P = int(chunk_page[n // PAGE])
        index_pages[P, :, :, kv_sel, n % PAGE, :] = idx[:, n, :, :]


def index_bytes_per_token(T: int, Tc: int, G: int, H: int, d: int) -> int:
    """Coded bytes per token and layer (K and V): one byte per (block, head, group, K/V)."""
    check_divisibility(T, Tc, G, d)
    return (T // Tc) * H * (d // (G // Tc)) * 2


# ----------------------------------------------------------------------------
# RoPE
# ----------------------------------------------------------------------------
def rope_inv_freq(d: int, base: float = 10000.0) -> np.ndarray:
    """theta_j = base^(-2j/d), j < d/2, float64."""
    return base ** (-2.0 * np.arange(d // 2, dtype=np.float64) / d)


def rope(x: np.ndarray, positions, base: float = 10000.0) -> np.ndarray:
    """Rotate-half RoPE in float64: pairs (j, j + d/2) turned by angle p * theta_j.

    x: ``[..., n, d]`` with positions ``[n]`` (or a scalar).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    ang = np.multiply.outer(np.asarray(positions, dtype=np.float64), rope_inv_freq(d, base))
    cos, sin = np.cos(ang), np.sin(ang)
    a, b = x[..., :d // 2], x[..., d // 2:]
    return np.concatenate([a * cos - b * sin, b * cos + a * sin], axis=-1)


# ----------------------------------------------------------------------------
# cache reconstruction and decode attention
# ----------------------------------------------------------------------------
@dataclass
class AttnShape:
    B: int
    H: int
    Hq: int
    d: int
    T: int
    Tc: int
    G: int
    n_sink: int
    rope_base: float = 10000.0
    scale: float = 0.0          # 0 -> 1/sqrt(d)

    @property
    def c(self):
        return self.G // self.Tc

    @property
    def ng(self):
        return self.d // self.c

    @property
    def nblk(self):
        return self.T // self.Tc

    @property
    def sm_scale(self):
        return self.scale if self.scale > 0 else 1.0 / np.sqrt(self.d)


def token_classes(L: int, q_end: int, n_sink: int) -> np.ndarray:
    """0 = sink (p < n_sink), 2 = recent (p >= q_end), 1 = coded; sink wins over recent."""
    p = np.arange(L)
    cls = np.where(p >= q_end, 2, 1)
    cls[p < n_sink] = 0
    return cls


def reconstruct_kv(shp: AttnShape, b: int, h: int, t: int, L: int, q_end: int,
                   page_table, index_pages, bf16_pages, bf16_table, cb) -> tuple[np.ndarray, np.ndarray]:
    """Pre-RoPE keys and values ``[L][d]`` (float64) of sequence b, KV head h, loop step t.

    bf16 tokens are read as stored.  A coded token takes, for every group g, the
    c-channel slice of step ``tau = t % Tc`` of the codeword its index row (block
    ``beta = t // Tc``) selects: only the step-t share is read (summary, section
    "전제와 한계"); values are reconstructed the same way (rit.work article,
    section "Когда LoopVQ меняет план развёртывания").
    cb: float64 codebooks ``[nblk][2][H][ng][Tc][256][c]``.
    """
    d, c, ng = shp.d, shp.c, shp.ng
    beta, tau = t // shp.Tc, t % shp.Tc
    K = np.zeros((L, d))
    V = np.zeros((L, d))
    cls = token_classes(L, q_end, shp.n_sink)
    p = np.arange(L)
    slot = p % PAGE
    # sink tokens: the retained bf16 copy of logical page 0
    sk = p[cls == 0]
    if len(sk):
        page = bf16_pages[bf16_table[b][0]]
        K[sk] = bf16_to_f64(page[t, h, 0, slot[sk]])
        V[sk] = bf16_to_f64(page[t, h, 1, slot[sk]])
    # recent tokens: bf16 pages listed in logical order from page q_end / 8
    rc = p[cls == 2]
    if len(rc):
        pages = np.asarray(bf16_table[b])[1 + rc // PAGE - q_end // PAGE]
        K[rc] = bf16_to_f64(bf16_pages[pages, t, h, 0, slot[rc]])
        V[rc] = bf16_to_f64(bf16_pages[pages, t, h, 1, slot[rc]])
    # coded tokens: group g of the token is the step-tau share of codeword row[g]
    cd = p[cls == 1]
    if len(cd):
        phys = np.asarray(page_table[b])[cd // PAGE]
        for kv, dst in ((0, K), (1, V)):
            rows = index_pages[phys, beta, h, kv, slot[cd]].astype(np.int64)   # [n][ng]
            book = cb[beta, kv, h, :, tau]                                       # [ng][256][c]
            dst[cd] = book[np.arange(ng)[None, :], rows].reshape(len(cd), ng * c)
    return K, V


def attend(qr: np.ndarray, Kr: np.ndarray, V: np.ndarray, scale: float):
    """Softmax attention of one rotated query over rotated keys: (out, lse, scores).

    With no keys (an empty sequence) the weighted sum and the sum of weights are both
    empty: the output is the zero vector and lse = log 0 = -inf (a reading; the pages
    do not speak of empty sequences).
    """
    if len(Kr) == 0:
        return np.zeros(V.shape[1]), -np.inf, np.zeros(0)
    s = (Kr @ qr) * scale
    m = s.max()
    w = np.exp(s - m)
    l = w.sum()
    return (w @ V) / l, m + np.log(l), s


def decode_attn(shp: AttnShape, q_bits, page_table, index_pages, bf16_pages, bf16_table,
                codebooks_bits, t: int, pos, seq_len, q_end, return_scores: bool = False,
                heads=None, pairs=None):
    """Decode attention at loop step t over the paged LoopVQ cache.

    Returns ``out[B][Hq][d]`` and ``lse[B][Hq]`` (float64) and optionally the
    scaled scores per (b, hq).  Query head hq reads KV head hq // (Hq / H).
    ``heads`` (query heads) or ``pairs`` ((b, hq) list) optionally restrict what is
    computed; the rest is NaN.
    """
    B, Hq, d = shp.B, shp.Hq, shp.d
    grp = Hq // shp.H
    cb = bf16_to_f64(codebooks_bits)
    q = bf16_to_f64(q_bits)
    out = np.full((B, Hq, d), np.nan)
    lse = np.full((B, Hq), np.nan)
    scores = {}
    cache = {}
    if pairs is None:
        pairs = [(b, hq) for b in range(B) for hq in (range(Hq) if heads is None else heads)]
    for b, hq in pairs:
        L = int(seq_len[b])
        h = hq // grp
        if (b, h) not in cache:
            K, V = reconstruct_kv(shp, b, h, t, L, int(q_end[b]), page_table, index_pages,
                                  bf16_pages, bf16_table, cb)
            cache[(b, h)] = (rope(K, np.arange(L), shp.rope_base), V)
        Kr, V = cache[(b, h)]
        qr = rope(q[b, hq], int(pos[b]), shp.rope_base)
        o, ls, s = attend(qr, Kr, V, shp.sm_scale)
        out[b, hq], lse[b, hq] = o, ls
        if return_scores:
            scores[(b, hq)] = s
    if return_scores:
        return out, lse, scores
    return out, lse


def split_partials(qr, Kr, V, scale, bounds):
    """(m, l, o) of each chunk ``[bounds[i], bounds[i+1])``; empty chunks give (-inf, 0, 0)."""
    parts = []
    s = (Kr @ qr) * scale
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        if hi <= lo:
            parts.append((-np.inf, 0.0, np.zeros(V.shape[1])))
            continue
        m = s[lo:hi].max()
        w = np.exp(s[lo:hi] - m)
        parts.append((m, w.sum(), w @ V[lo:hi]))
    return parts


def lse_merge(parts):
    """Merge chunk partials: m = max m_i, l = sum l_i e^(m_i - m), o = sum o_i e^(m_i - m) / l."""
    m = max(p[0] for p in parts)
    l = sum(p[1] * np.exp(p[0] - m) for p in parts if p[1] > 0)
    o = sum(p[2] * np.exp(p[0] - m) for p in parts if p[1] > 0)
    return o / l, m + np.log(l)


def decode_attn_split(shp: AttnShape, q_bits, page_table, index_pages, bf16_pages, bf16_table,
                      codebooks_bits, t: int, pos, seq_len, q_end, n_splits: int):
    """Flash-Decoding form: the coded range cut into ``n_splits`` contiguous chunks plus
    one chunk holding every bf16 token, merged by log-sum-exp (summary, section "전제와 한계")."""
    B, Hq, d = shp.B, shp.Hq, shp.d
    grp = Hq // shp.H
    cb = bf16_to_f64(codebooks_bits)
    q = bf16_to_f64(q_bits)
    out = np.zeros((B, Hq, d))
    lse = np.zeros((B, Hq))
    for b in range(B):
        L, qe = int(seq_len[b]), int(q_end[b])
        cls = token_classes(L, qe, shp.n_sink)
        coded = np.nonzero(cls == 1)[0]
        bf = np.nonzero(cls != 1)[0]
        for hq in range(Hq):
            h = hq // grp
            K, V = reconstruct_kv(shp, b, h, t, L, qe, page_table, index_pages, bf16_pages,
                                  bf16_table, cb)
            Kr = rope(K, np.arange(L), shp.rope_base)
            qr = rope(q[b, hq], int(pos[b]), shp.rope_base)
            order = np.concatenate([coded, bf])
            n_c = len(coded)
            cuts = [round(i * n_c / n_splits) for i in range(n_splits + 1)] + [n_c + len(bf)]
            parts = split_partials(qr, Kr[order], V[order], shp.sm_scale, cuts)
            out[b, hq], lse[b, hq] = lse_merge(parts)
    return out, lse


def needle_mass(scores: np.ndarray, lse: float, lo: int, hi: int) -> float:
    """Attention mass on positions [lo, hi): sum of exp(s_p - lse)."""
    return float(np.exp(scores[lo:hi] - lse).sum())


# ----------------------------------------------------------------------------
# codebook builder: k-means++ seeding and Lloyd iterations
# ----------------------------------------------------------------------------
# The summary (section "전제와 한계", experiments paragraph) calibrates the
# codebooks by k-means on calibration K/V, and (section "무엇과 다른가") initialises
# them by Fisher-weighted k-means; the pages fix neither the seeding, the weights nor the precision.
# Readings: one non-negative weight per joint vector, given as an input (the Fisher
# information itself needs model gradients); k-means++ seeding (weighted D^2
# sampling) driven by draws passed in; Lloyd iterations whose assignment uses the
# centers rounded to bf16 (the stored codebook precision, so the assignment is
# exactly the encoder's nearest codeword) and whose update is the float64 weighted
# mean of the members taken in sample order, a cluster of zero total weight keeping
# its center; the final centers rounded to bf16 (via float32, round to nearest even).

def round_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> float32 (round to nearest even) -> bf16 (round to nearest even), as float64."""
    bits = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32)).view(np.uint32)
    bits = bits.astype(np.uint64)
    rounded = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16).astype(np.uint16)
    return bf16_to_f64(rounded)


def bf16_bits_of(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of float64 values that are exactly bf16."""
    return (np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32) >> 16).astype(np.uint16)


def sq_dist_sequential(X: np.ndarray, c: np.ndarray) -> np.ndarray:
    """sum_e (X[s][e] - c[e])^2 for every s, adding the squares in order e = 0, 1, ..."""
    d = np.zeros(X.shape[0])
    for e in range(X.shape[1]):
        df = X[:, e] - c[e]
        d = d + df * df
    return d


def _running_sum_pick(terms: np.ndarray, u: float) -> int:
    """The first s whose running sum terms_0 + ... + terms_s (sample order) exceeds
    u times the total; the last s with a positive term if rounding leaves none; sample
    floor(u * S) if the total is not positive."""
    S = terms.shape[0]
    cum = np.cumsum(terms)
    total = cum[-1]
    if total > 0:
        above = np.flatnonzero(cum > u * total)
        return int(above[0]) if len(above) else int(np.flatnonzero(terms > 0)[-1])
    return min(max(int(u * S), 0), S - 1)


def kmeanspp_seed(X: np.ndarray, draws: np.ndarray, K: int = NCODES, w=None) -> np.ndarray:
    """k-means++ seeding: indices of the K samples chosen as initial centers.

    Sample s carries weight w_s (1 when ``w`` is None).  Draw 0 picks by weight alone
    (every distance taken as 1), which is sample floor(u_0 * S) without weights.  Draw
    k >= 1 picks by the terms w_s * D^2_s, D^2_s being the squared distance of sample
    s to its nearest chosen center.  Each pick is ``_running_sum_pick``: running sums
    in sample order compared with u_k times the total.
    """
    S = X.shape[0]
    wv = np.ones(S) if w is None else np.asarray(w, dtype=np.float64)
    picks = np.empty(K, dtype=np.int64)
    picks[0] = _running_sum_pick(wv, draws[0])
    D2 = sq_dist_sequential(X, X[picks[0]])
    for k in range(1, K):
        i = _running_sum_pick(wv * D2, draws[k])
        picks[k] = i
        D2 = np.minimum(D2, sq_dist_sequential(X, X[i]))
    return picks


def lloyd(X: np.ndarray, centers: np.ndarray, n_iter: int, bf16_assign: bool = True, w=None) -> np.ndarray:
    """n_iter Lloyd iterations from ``centers`` (float64 [K][G]).

    Assignment: nearest center by squared L2, lowest index on ties, against the
    centers rounded to bf16 (``bf16_assign``) or as they are.  Update: the weighted
    mean sum(w_s x_s) / sum(w_s) of each cluster's members (w_s = 1 when ``w`` is
    None), both sums in sample order; a cluster whose weights sum to 0 (an empty one
    in particular) keeps its center.
    """
    C = np.array(centers, dtype=np.float64)
    K, G = C.shape
    wv = None if w is None else np.asarray(w, dtype=np.float64)
    for _ in range(n_iter):
        A = round_bf16(C) if bf16_assign else C
        assign = nearest_codeword(X, A).idx
        new = C.copy()
        for k in range(K):
            acc = np.zeros(G)
            wsum = 0.0
            for s in np.flatnonzero(assign == k):
                if wv is None:
                    acc = acc + X[s]
                    wsum = wsum + 1.0
                else:
                    acc = acc + wv[s] * X[s]
                    wsum = wsum + wv[s]
            if wsum != 0.0:
                new[k] = acc / wsum
        C = new
    return C


def build_codebooks(samples_bits: np.ndarray, draws: np.ndarray, Tc: int, G: int, n_iter: int,
                    books=None, weights=None) -> np.ndarray:
    """Codebooks of one of K / V: ``samples[T][S][H][d]`` (bf16) -> bf16 bits ``[nblk][H][ng][Tc][256][c]``.

    draws: ``[nblk][H][ng][256]`` uniform numbers in [0, 1).  Book (beta, h, g) is
    trained on the joint vectors of its (block, head, group) over the S samples, with
    the per-vector weights ``weights[beta][s][h][g]`` (float64 [nblk][S][H][ng]; None =
    all 1), k-means++ seeding and ``n_iter`` Lloyd iterations, then rounded to bf16.
    ``books`` optionally restricts the work to a list of (beta, h, g); the rest stays 0.
    """
    X = bf16_to_f64(samples_bits)
    T, S, H, d = X.shape
    J = joint_vectors(X, Tc, G)                 # [nblk][S][H][ng][G]
    nblk, ng, c = T // Tc, d // (G // Tc), G // Tc
    out = np.zeros((nblk, H, ng, Tc, NCODES, c), dtype=np.uint16)
    todo = books if books is not None else [(b, h, g) for b in range(nblk) for h in range(H) for g in range(ng)]
    for beta, h, g in todo:
        x = J[beta, :, h, g]
        w = None if weights is None else weights[beta, :, h, g]
        picks = kmeanspp_seed(x, draws[beta, h, g], w=w)
        C = lloyd(x, x[picks], n_iter, w=w)
        Cb = bf16_bits_of(round_bf16(C))            # [256][G]
        for tau in range(Tc):
            out[beta, h, g, tau] = Cb[:, tau * c:(tau + 1) * c]
    return out


# ----------------------------------------------------------------------------
# paged cache bookkeeping
# ----------------------------------------------------------------------------
# The summary (section "전제와 한계") keeps the sink and the recent window in bf16,
# pages the cache in 8 tokens, and once a token's forward pass is over quantises the
# oldest recent page (all layers and loop steps) every 8 tokens.  Readings: after
# prefill the coded run ends at q_end = 8 floor((L - n_recent) / 8) (0 when negative);
# after each decode token, with L tokens cached, the oldest recent page is coded when
# L - q_end >= n_recent + 8.

def prefill_boundary(L: int, n_recent: int) -> int:
    """q_end right after a prefill of L tokens."""
    return max(0, PAGE * ((L - n_recent) // PAGE))


def decode_boundary(q_end: int, L: int, n_recent: int) -> int:
    """q_end after the forward pass of the token that brought the cache to L tokens."""
    return q_end + PAGE if L - q_end >= n_recent + PAGE else q_end
