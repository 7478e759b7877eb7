"""Pins of the oracle's sampled verification.

* Philox-4x32-10 against the known-answer vectors published with the Random123 library
  (the reference implementation of the SC 2011 paper that defines the generator).
* Uniforms lie strictly inside (0, 1) and are statistically uniform.
* The Gumbel-max sample follows softmax(logits / T): chi-square over many draws.
* T -> 0 gives the argmax; a planted +16 logit is always drawn at T = 1.
"""

import numpy as np
import pytest

import oracle

KAT = [  # (counter c0..c3, key k0 k1) -> output words, philox4x32 with 10 rounds
    ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF, 0xFFFFFFFF), (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


@pytest.mark.parametrize("ctr,key,expect", KAT)
def test_philox_known_answers(ctr, key, expect):
    out = oracle.philox4x32_10(ctr, key)
    assert tuple(int(w) for w in out) == expect


def test_uniforms_in_open_interval_and_uniform():
    u = oracle.uniforms(4, 50000, seed=1234, offset=7)
    assert u.min() > 0 and u.max() < 1
    assert np.array_equal(u.astype(np.float32).astype(np.float64), u)   # exact in float32
    hist, _ = np.histogram(u.ravel(), bins=20, range=(0, 1))
    expected = u.size / 20
    chi2 = ((hist - expected) ** 2 / expected).sum()
    assert chi2 < 45          # 19 dof: p ~ 0.001
    # different seeds / offsets / nodes give different streams
    assert not np.array_equal(u[0], u[1])
    assert not np.array_equal(oracle.uniforms(1, 64, 1234, 8)[0], u[0, :64])


def test_gumbel_max_follows_softmax():
    logits = np.array([[0.0, 1.0, -0.5, 2.0, 0.3, -2.0, 1.5, 0.0]])
    T = 0.7
    p = np.exp(logits[0] / T - (logits[0] / T).max())
    p /= p.sum()
    n = 20000
    counts = np.zeros(8)
    for off in range(n):
        counts[oracle.sample_rows(logits, T, seed=99, offset=off)[0]] += 1
    chi2 = ((counts - n * p) ** 2 / (n * p)).sum()
    assert chi2 < 24          # 7 dof: p ~ 0.001


def test_low_temperature_is_argmax_and_planted_token_wins():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((6, 1000))
    assert np.array_equal(oracle.sample_rows(x, 1e-4, 3, 0), oracle.argmax_rows(x))
    x[np.arange(6), [5, 17, 900, 0, 999, 321]] = 16.0
    for off in range(20):
        assert oracle.sample_rows(x, 1.0, 11, off).tolist() == [5, 17, 900, 0, 999, 321]


def test_sample_accept_uses_the_sampled_tokens():
    rng = np.random.default_rng(8)
    parent = np.array([-1, 0, 1, 1, 3], dtype=np.int32)
    x = rng.standard_normal((5, 40))
    tok, (m, nodes, toks, bonus) = oracle.sample_accept(parent, np.zeros(5, np.int64), x, 0.9, 1, 2)
    assert np.array_equal(tok, oracle.sample_rows(x, 0.9, 1, 2))
    m2, nodes2, _, bonus2 = oracle.accept(parent, tok, tok)
    assert m2 == 4 and nodes2.tolist() == [0, 1, 3, 4]
    with pytest.raises(ValueError):
        oracle.sample_rows(x, 0.0, 1, 2)
