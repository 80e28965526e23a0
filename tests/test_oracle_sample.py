"""Pins of the oracle's sampled draw (CPU only): Philox4x32-10 against the published
known-answer vectors, the uniform's distribution, the reductions to the greedy argmax, and
the filtered softmax by chi-squared tests over many positions.

The draw (Strata docs/BATCHING.md, "Exactness": sampled rows are drawn one by one with the
single-request window's counter-based draw, Philox(seed, position)); the generator is
Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC'11), whose
reference implementation publishes the known-answer vectors checked here."""
import numpy as np
import pytest
from scipy import stats


@pytest.fixture(scope="module")
def orc(oracle_lib):
    return oracle_lib


@pytest.mark.parametrize("ctr,key,want", [
    ([0, 0, 0, 0], [0, 0], [0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8]),
    ([0xffffffff] * 4, [0xffffffff] * 2, [0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd]),
    ([0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344], [0xa4093822, 0x299f31d0],
     [0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1]),
])
def test_philox_known_answers(orc, ctr, key, want):
    assert [int(v) for v in orc.philox4x32_10(ctr, key)] == want


def test_uniform_distribution(orc):
    u = np.array([orc.uniform(12345, p) for p in range(20000)])
    assert u.min() >= 0.0 and u.max() < 1.0
    assert stats.kstest(u, "uniform").pvalue > 1e-4
    # another seed gives another, uncorrelated sequence
    v = np.array([orc.uniform(54321, p) for p in range(20000)])
    assert abs(np.corrcoef(u, v)[0, 1]) < 0.05
    # the uniform is the first two output words as a 53-bit fraction
    o = orc.philox4x32_10([7, 0, 0, 0], [9, 0])
    assert orc.uniform(9, 7) == (int(o[0]) * 2**21 + (int(o[1]) >> 11)) / 2**53


def _softmax(l, T):
    z = (l.astype(np.float64) - l.max()) / T
    p = np.exp(z)
    return p / p.sum()


def test_greedy_reductions(orc):
    rng = np.random.default_rng(1)
    for trial in range(20):
        V = int(rng.integers(2, 3000))
        l = rng.standard_normal(V).astype(np.float32)
        if trial % 4 == 0:   # ties: the lowest index of the largest value
            l[rng.integers(0, V, 5)] = l.max()
        am = int(np.argmax(l))
        # temperature 0: greedy, whatever the other parameters and the draw
        assert orc.sample(l, 0.0, 40, 0.9, 0.05, seed=trial, position=trial)[0] == am
        # top_k 1: the argmax at any temperature
        assert orc.sample(l, 1.3, 1, 1.0, 0.0, seed=trial, position=5)[0] == am
        # a temperature far below the top-two gap leaves all the mass on the largest logit
        s = np.sort(l)[::-1]
        if s[0] > s[1]:
            assert orc.sample(l, float(s[0] - s[1]) / 1000.0, 128, 1.0, 0.0, seed=trial, position=3)[0] == am


def _draws(orc, l, T, k, top_p, min_p, n, seed=77):
    return np.array([orc.sample(l, T, k, top_p, min_p, seed=seed, position=p)[0] for p in range(n)])


def test_chi_squared_full_softmax(orc):
    rng = np.random.default_rng(2)
    l = (rng.standard_normal(48) * 1.5).astype(np.float32)
    for T in (1.0, 2.0):
        d = _draws(orc, l, T, 128, 1.0, 0.0, 30000)
        p = _softmax(l, T)
        obs = np.bincount(d, minlength=48)
        keep = p * len(d) >= 5   # bins with enough expected counts; the rest pooled
        o, e = obs[keep], p[keep] * len(d)
        if (~keep).any():
            o, e = np.append(o, obs[~keep].sum()), np.append(e, p[~keep].sum() * len(d))
        assert stats.chisquare(o, e).pvalue > 1e-4, T


def test_top_k_draws_only_candidates(orc):
    rng = np.random.default_rng(3)
    l = rng.standard_normal(500).astype(np.float32)
    d = _draws(orc, l, 1.0, 7, 1.0, 0.0, 6000)
    top = np.argsort(-l, kind="stable")[:7]
    assert set(d) <= set(top)
    p = _softmax(l[top], 1.0)
    obs = np.array([(d == t).sum() for t in top])
    assert stats.chisquare(obs, p * len(d)).pvalue > 1e-4


@pytest.mark.parametrize("kw", [dict(top_p=0.7, min_p=0.0), dict(top_p=1.0, min_p=0.3)])
def test_top_p_and_min_p_hand_case(orc, kw):
    """Probabilities 1/2, 1/4, 1/8, 1/16, 1/16: top_p 0.7 keeps the first two (1/2 < 0.7 <=
    3/4), and min_p 0.3 keeps those at or above 0.3 x 1/2, the same two; draws then go 2:1."""
    l = np.log(np.array([0.5, 0.25, 0.125, 0.0625, 0.0625])).astype(np.float32)
    d = _draws(orc, l, 1.0, 5, kw["top_p"], kw["min_p"], 9000)
    assert set(d) <= {0, 1}
    n0 = (d == 0).sum()
    assert stats.binomtest(int(n0), len(d), 2 / 3).pvalue > 1e-4


def test_sampled_verify_is_the_greedy_rule_with_draws(orc):
    """A slot keeps its proposal when it equals the draw of its token row, then emits the
    draw of the proposal row: the greedy accept with each row's draw for its argmax."""
    rng = np.random.default_rng(4)
    R, V = 8, 300
    l = rng.standard_normal((R, V)).astype(np.float32)
    pos = np.array([100, 101, 250, 251, 7, 8, 40, 41])
    draws = np.array([orc.sample(l[r], 0.8, 50, 0.95, 0.02, seed=900 + r // 2, position=pos[r])[0]
                      for r in range(R)], np.int32)
    prop = draws[0::2].copy()
    prop[1] += 1          # one proposal differs from its slot's draw
    tokens, n_tok, kept = orc.accept(draws, prop, mtp=True)
    assert kept == 3
    assert list(n_tok) == [2, 1, 2, 2]
    assert tokens[0].tolist() == [draws[0], draws[1]] and tokens[1].tolist() == [draws[2], -1]
