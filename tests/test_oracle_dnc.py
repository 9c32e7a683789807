"""Pins of the integer-exact numerics contract (oracle/dnc.py) against published definitions,
error bounds, statistics and brute force.  CPU only."""
import itertools
import math
import os

import numpy as np
import pytest
from scipy import stats

from oracle import dnc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _ulp32(x):
    x = np.abs(np.asarray(x, np.float32))
    return np.spacing(x).astype(np.float64)


def test_splitmix64_published_vector():
    vals = [int(l, 16) for l in open(os.path.join(GOLDEN, "splitmix64_seed0.txt"))
            if l.strip() and not l.startswith("#")]
    state = 0
    for v in vals:
        state = (state + dnc.GOLDEN) % (1 << 64)
        assert dnc.mix64(state) == v


def test_constants_follow_their_definitions():
    # LN2_HI: 16 significant bits, so k * LN2_HI is exact for |k| <= 128
    bits = int(np.frombuffer(dnc.LN2_HI.tobytes(), np.uint32)[0])
    assert bits & 0xFF == 0
    # LN2_LO is ln 2 - LN2_HI rounded to fp32: within half an fp32 ulp of the exact remainder
    assert abs(float(dnc.LN2_HI) + float(dnc.LN2_LO) - math.log(2.0)) <= 0.5 * float(
        np.spacing(dnc.LN2_LO)) + 1e-16
    for k in range(-128, 129):
        assert float(np.float32(k) * dnc.LN2_HI) == k * float(dnc.LN2_HI)
    for i, c in enumerate(dnc.TAYLOR):
        assert float(c) == float(np.float32(1.0 / math.factorial(i)))
    assert abs(float(dnc.LOG2E) - 1 / math.log(2)) < 1e-7


def test_exp_dnc_error_bound_against_exp():
    rng = np.random.default_rng(1)
    x = np.concatenate([-rng.exponential(8.0, 400_000), -rng.random(100_000) * 44.0,
                        np.array([0.0, -1e-30, -1e-7, -0.5, -1.0, -43.9, -44.0])]).astype(
        np.float32)
    got = dnc.exp_dnc(x).astype(np.float64)
    ref = np.exp(x.astype(np.float64))
    keep = x.astype(np.float64) * (1 / math.log(2)) >= -63.5     # away from the cut-off
    err = np.abs(got - ref)[keep] / _ulp32(ref[keep].astype(np.float32))
    assert err.max() <= 2.0, err.max()


def test_exp_dnc_special_values():
    assert dnc.exp_dnc(np.float32(0.0)) == np.float32(1.0)
    # near powers of two: x = fp32(-k ln 2) reduces to k with a tiny remainder r
    for k in range(0, 60):
        x = np.float32(-k * math.log(2.0))
        v = float(dnc.exp_dnc(x))
        assert abs(v / math.exp(float(x)) - 1) < 2.4e-7
    assert dnc.exp_dnc(np.float32(-100.0)) == 0.0          # below the cut-off
    assert np.all(np.diff(dnc.exp_dnc(np.linspace(-40, 0, 20001, dtype=np.float32))) >= 0)


def test_argmax_lowest_on_planted_ties():
    rng = np.random.default_rng(2)
    for V in (1, 2, 7, 64, 1000):
        for _ in range(50):
            row = rng.integers(-3, 4, size=V).astype(np.float32)   # many exact ties
            brute = min(i for i in range(V) if row[i] == row.max())
            assert dnc.argmax_lowest(row) == brute
    row = np.array([-0.0, 0.0, -1.0], np.float32)                   # +0 == -0
    assert dnc.argmax_lowest(row) == 0


def test_row_weights_exact_integers():
    row = np.array([0.0, -1.0, -2.0, 5.0, 5.0, -200.0], np.float32)
    q, Z = dnc.row_weights(row)
    assert int(q[3]) == 1 << 40 and int(q[4]) == 1 << 40     # exp_dnc(0) = 1 exactly
    assert int(q[5]) == 0                                     # below 2^-40
    assert Z == sum(int(v) for v in q)                        # exact integer sum
    e = np.exp(row.astype(np.float64) - 5.0)
    assert np.all(np.abs(q.astype(np.float64) / 2.0 ** 40 - e) <= 2.0 ** -40 + 2.4e-7 * e)


def test_sample_token_brute_force():
    rng = np.random.default_rng(3)
    for _ in range(200):
        V = int(rng.integers(1, 9))
        q = rng.integers(0, 5, size=V).astype(np.uint64)
        if int(q.sum()) == 0:
            q[int(rng.integers(0, V))] = 1
        Z = int(q.sum())
        for u in (0, 1, 12345, (1 << 31), (1 << 32) - 1, int(rng.integers(0, 1 << 32))):
            thr = (u * Z) >> 32
            brute = next(v for v in range(V) if sum(int(x) for x in q[: v + 1]) > thr)
            assert dnc.sample_token(q, Z, u) == brute
            assert int(q[brute]) > 0                          # zero-weight tokens never drawn


@pytest.mark.parametrize("V,T", [(8, 1.0), (8, 1.5), (64, 1.0), (64, 1.5)])
def test_sampler_chi_square(V, T):
    rng = np.random.default_rng(V * 10 + int(T * 10))
    logits = (rng.standard_normal(V) * 2.0).astype(np.float32)
    q, Z = dnc.row_weights(logits, dnc.inv_temperature(T))
    n = 40_000
    draws = np.array([dnc.sample_token(q, Z, dnc.draw_u32(7, 0, 0, j, 1, n)) for j in range(n)])
    p = np.exp(logits.astype(np.float64) / T - (logits.max() / T))
    p /= p.sum()
    counts = np.bincount(draws, minlength=V)
    big = p * n >= 5
    obs = np.append(counts[big], counts[~big].sum())
    exp = np.append(p[big] * n, p[~big].sum() * n)
    if exp[-1] == 0:
        obs, exp = obs[:-1], exp[:-1]
    chi2 = ((obs - exp) ** 2 / exp).sum()
    pval = stats.chi2.sf(chi2, len(obs) - 1)
    assert pval > 1e-4, (chi2, pval)


def test_k_drafts_are_independent():
    V, K, n = 6, 2, 30_000
    rng = np.random.default_rng(5)
    logits = (rng.standard_normal(V)).astype(np.float32)
    q, Z = dnc.row_weights(logits)
    a = np.array([dnc.sample_token(q, Z, dnc.draw_u32(11, i, 0, 0, K, 1)) for i in range(n)])
    b = np.array([dnc.sample_token(q, Z, dnc.draw_u32(11, i, 1, 0, K, 1)) for i in range(n)])
    table = np.zeros((V, V))
    np.add.at(table, (a, b), 1)
    table = table[table.sum(1) > 0][:, table.sum(0) > 0]
    _, pval, _, _ = stats.chi2_contingency(table)
    assert pval > 1e-4


def test_token_prob_close_to_exact_softmax():
    rng = np.random.default_rng(6)
    for V in (10, 1000, 50_000):
        row = (rng.standard_normal(V) * 2).astype(np.float32)
        p_exact = np.exp(row.astype(np.float64) - row.max())
        p_exact /= p_exact.sum()
        for tok in rng.integers(0, V, size=20):
            p = dnc.token_prob(row, int(tok))
            assert abs(p - p_exact[tok]) <= 1e-6 * p_exact[tok] + V * 2.0 ** -40


def test_sample_drafts_argmax_mode_and_shapes():
    rng = np.random.default_rng(8)
    lg = rng.standard_normal((2, 3, 17)).astype(np.float32)
    out = dnc.sample_drafts(lg, 1, 0.0, 0)
    assert out.shape == (2, 1, 3)
    assert np.array_equal(out[:, 0, :], lg.argmax(-1))
    s = dnc.sample_drafts(lg, 4, 1.5, 123)
    assert s.shape == (2, 4, 3) and s.min() >= 0 and s.max() < 17
    assert np.array_equal(s, dnc.sample_drafts(lg, 4, 1.5, 123))   # pure function of the seed


# ---- top-p nucleus filter ----

def test_top_p_nucleus_is_a_smallest_heaviest_set_brute_force():
    """Against every subset of a tiny vocabulary: the nucleus reaches ceil(p Z), no smaller subset
    does, every token outside it weighs no more than every token inside, and among equal
    weights the lower indices are inside."""
    rng = np.random.default_rng(4)
    for _ in range(60):
        V = int(rng.integers(2, 9))
        logits = rng.integers(-4, 3, V).astype(np.float32) * np.float32(0.5)   # planted ties
        q, Z = dnc.row_weights(logits)
        p = float(np.float32(rng.uniform(0.05, 0.999)))
        need = dnc.top_p_threshold(Z, p)
        w = dnc.nucleus_weights(q, Z, p)
        inside = [v for v in range(V) if w[v] > 0]
        assert sum(int(q[v]) for v in inside) >= need
        best = min(len(S) for r in range(1, V + 1) for S in itertools.combinations(range(V), r)
                   if sum(int(q[v]) for v in S) >= need)
        assert len(inside) == best
        outside = [v for v in range(V) if w[v] == 0]
        if outside and inside:
            assert max(int(q[v]) for v in outside) <= min(int(q[v]) for v in inside)
        for a in inside:
            for b in outside:
                if int(q[a]) == int(q[b]):
                    assert a < b


def test_top_p_threshold_is_the_exact_ceiling():
    from fractions import Fraction
    for Z in (1, 7, 1 << 40, (1 << 57) + 12345):
        for p in (0.5, 0.9, 0.25, 1e-7, 0.3):
            pf = Fraction(float(np.float32(p)))
            t = dnc.top_p_threshold(Z, p)
            assert t - 1 < pf * Z <= t


def test_top_p_one_is_plain_sampling_and_tiny_p_is_argmax():
    rng = np.random.default_rng(5)
    logits = (rng.normal(size=(3, 4, 50)) * 2).astype(np.float32)
    a = dnc.sample_drafts(logits, 4, 1.3, seed=8)
    b = dnc.sample_drafts(logits, 4, 1.3, seed=8, top_p=1.0)
    assert np.array_equal(a, b)
    c = dnc.sample_drafts(logits, 4, 1.3, seed=8, top_p=1e-6)
    assert np.array_equal(c, np.broadcast_to(logits.argmax(-1)[:, None, :], c.shape))


@pytest.mark.parametrize("p", [0.6, 0.9])
def test_top_p_sampler_chi_square(p):
    """Draws restricted to the nucleus follow the fp64 softmax renormalised over it (the nucleus
    boundary is away from p here, so fp64 and the integer weights select the same set)."""
    from scipy import stats
    V, n = 16, 20_000
    logits = np.linspace(2.0, -2.0, V).astype(np.float32)
    P = np.exp(logits.astype(np.float64) - logits.max())
    P /= P.sum()
    cum = np.cumsum(np.sort(P)[::-1])
    k = int(np.searchsorted(cum, p) + 1)
    assert min(abs(cum - p)) > 1e-3
    keep = np.argsort(-P, kind="stable")[:k]
    Pn = np.zeros(V)
    Pn[keep] = P[keep] / P[keep].sum()
    rows = np.broadcast_to(logits, (n, 1, V)).copy()
    toks = dnc.sample_drafts(rows, 1, 1.0, seed=3, top_p=p)[:, 0, 0]
    counts = np.bincount(toks, minlength=V)
    assert counts[Pn == 0].sum() == 0
    sel = Pn > 0
    chi2 = float(((counts[sel] - n * Pn[sel]) ** 2 / (n * Pn[sel])).sum())
    assert chi2 < stats.chi2.ppf(1 - 1e-4, int(sel.sum()) - 1), chi2
