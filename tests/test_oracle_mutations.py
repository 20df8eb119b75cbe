"""Plant plausible mistakes in the oracle (on the CPU) and check that a pin catches each.

This is what makes the pins trustworthy: every mutant below must make at least
one pin in test_oracle_pins fail.
"""
import numpy as np
import pytest

import test_oracle_pins as pins
from oracle import lvq_oracle as orc

PINS = [
    pins.test_p9_nearest_matches_scipy_vq,
    pins.test_p9_tiny_hand_cases,
    pins.test_p11_duplicate_codewords_lowest_index,
    pins.test_p3_product_codebook_separates,
    pins.test_p2_tc1_is_per_step_coding,
    lambda: pins.test_p4_all_bf16_is_textbook_attention(37, 4),
    lambda: pins.test_p5_identity_codebook_end_to_end(2, 16),
    lambda: pins.test_p5_identity_codebook_end_to_end(4, 32),
    pins.test_p6_lse_merge_equals_unsplit,
    pins.test_p7_step_slice_locality,
    pins.test_p10_rope_relative_invariance_and_closed_forms,
    pins.test_p12_single_token,
    pins.test_boundary_conventions,
]


def _caught() -> bool:
    for pin in PINS:
        try:
            pin()
        except (AssertionError, IndexError, ValueError):
            return True
    return False


def _rope_sign_flipped(x, positions, base=10000.0):
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    ang = np.multiply.outer(np.asarray(positions, dtype=np.float64), orc.rope_inv_freq(d, base))
    a, b = x[..., :d // 2], x[..., d // 2:]
    return np.concatenate([a * np.cos(ang) + b * np.sin(ang), b * np.cos(ang) - a * np.sin(ang)], -1)


def _rope_interleaved(x, positions, base=10000.0):
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    ang = np.multiply.outer(np.asarray(positions, dtype=np.float64), orc.rope_inv_freq(d, base))
    a, b = x[..., 0::2], x[..., 1::2]
    out = np.empty(np.broadcast_shapes(x.shape, ang.shape[:-1] + (d,)))
    out[..., 0::2] = a * np.cos(ang) - b * np.sin(ang)
    out[..., 1::2] = b * np.cos(ang) + a * np.sin(ang)
    return out


def _rope_wrong_freq(x, positions, base=10000.0):
    return orc_rope_orig(x, positions, base * 2)


def _joint_channel_major(X, Tc, G):
    T, N, H, d = X.shape
    c = G // Tc
    nblk, ng = T // Tc, d // c
    out = np.empty((nblk, N, H, ng, G))
    for beta in range(nblk):
        for tau in range(Tc):
            for g in range(ng):
                out[beta, :, :, g, tau::Tc] = X[beta * Tc + tau][:, :, g * c:(g + 1) * c]
    return out


def _nearest_last_index(x, C, chunk=1024):
    r = orc_nearest_orig(x, C, chunk)
    D = ((x[:, None, :] - C[None]) ** 2).sum(-1)
    r.idx = (C.shape[0] - 1) - np.argmin(D[:, ::-1], axis=1)
    return r


def _nearest_dot_only(x, C, chunk=1024):
    # drops the |C|^2 term: picks the largest inner product
    r = orc_nearest_orig(x, C, chunk)
    r.idx = np.argmax(x @ C.T, axis=1)
    return r


def _attend_no_scale(qr, Kr, V, scale):
    return orc_attend_orig(qr, Kr, V, 1.0)


def _merge_no_rescale(parts):
    m = max(p[0] for p in parts)
    l = sum(p[1] for p in parts if p[1] > 0)
    o = sum(p[2] for p in parts if p[1] > 0)
    return o / l, m + np.log(l)


def _classes_recent_wins(L, q_end, n_sink):
    p = np.arange(L)
    cls = np.ones(L, dtype=int)
    cls[p < n_sink] = 0
    cls[p >= q_end] = 2
    return cls


def _classes_drop_last_recent(L, q_end, n_sink):
    cls = orc_classes_orig(L, q_end, n_sink)
    return cls[:-1] if L > 1 else cls


orc_rope_orig = orc.rope
orc_nearest_orig = orc.nearest_codeword
orc_attend_orig = orc.attend
orc_classes_orig = orc.token_classes


def _reconstruct_step_from_block_start(shp, b, h, t, L, q_end, *a):
    return orc_reconstruct_orig(shp, b, h, (t // shp.Tc) * shp.Tc, L, q_end, *a)


orc_reconstruct_orig = orc.reconstruct_kv

MUTANTS = {
    "rope_sign": ("rope", _rope_sign_flipped),
    "rope_interleaved_pairs": ("rope", _rope_interleaved),
    "rope_base": ("rope", _rope_wrong_freq),
    "joint_channel_major": ("joint_vectors", _joint_channel_major),
    "ties_last_index": ("nearest_codeword", _nearest_last_index),
    "distance_drops_norm": ("nearest_codeword", _nearest_dot_only),
    "no_softmax_scale": ("attend", _attend_no_scale),
    "merge_no_rescale": ("lse_merge", _merge_no_rescale),
    "recent_overrides_sink": ("token_classes", _classes_recent_wins),
    "wrong_step_slice": ("reconstruct_kv", _reconstruct_step_from_block_start),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(orc, attr, fn)
    assert _caught(), f"no pin caught mutant {name}"
