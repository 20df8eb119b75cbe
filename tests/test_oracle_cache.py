"""Pins of the paged-cache bookkeeping rules of the oracle (prefill boundary, decode-time
re-encode trigger)."""
import pytest

from oracle import lvq_oracle as orc


def test_boundary_values_of_the_workloads():
    # tiny case: 512 tokens, 4 sink and 16 recent bf16 -> 492 coded tokens, so q_end = 496
    assert orc.prefill_boundary(512, 16) == 496
    assert orc.prefill_boundary(512, 16) - 4 == 492
    # Ouro-shaped: 32768 tokens with 64 recent -> 32704 (4088 coded pages)
    assert orc.prefill_boundary(32768, 64) == 32704
    # shorter than the window: nothing coded
    assert orc.prefill_boundary(60, 64) == 0
    assert orc.prefill_boundary(71, 64) == 0
    assert orc.prefill_boundary(72, 64) == 8


@pytest.mark.parametrize("n_recent", [0, 5, 16, 64])
@pytest.mark.parametrize("L0", [1, 7, 8, 63, 64, 100, 517])
def test_decode_rule_keeps_the_window_between_n_recent_and_n_recent_plus_8(L0, n_recent):
    # the step rule applied token by token agrees with the prefill formula at every length,
    # i.e. the window r = L - q_end stays in [n_recent, n_recent + 8) once L >= n_recent
    q = orc.prefill_boundary(L0, n_recent)
    for L in range(L0 + 1, L0 + 200):
        q = orc.decode_boundary(q, L, n_recent)
        assert q == orc.prefill_boundary(L, n_recent)
        r = L - q
        assert q % 8 == 0
        assert r < n_recent + 8
        assert r >= n_recent or q == 0


def test_trigger_mutant_is_caught(monkeypatch):
    """'>' for '>=' in the trigger lets the window reach n_recent + 8 after a step."""
    monkeypatch.setattr(orc, "decode_boundary",
                        lambda q, L, n: q + 8 if L - q > n + 8 else q)
    with pytest.raises(AssertionError):
        test_decode_rule_keeps_the_window_between_n_recent_and_n_recent_plus_8(64, 16)
