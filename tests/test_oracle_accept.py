"""Pins of the acceptance / selection oracle (oracle/accept.py): closed forms, Monte Carlo,
enumeration and brute force on tiny vocabularies.  CPU only."""
import itertools

import numpy as np
import pytest

from oracle import accept, dnc
import synth


def _brute_greedy(logits, draft):
    """Independent brute force: t_j by scanning for the first strict maximum; the accepted count
    is the largest a such that every j < a matches."""
    R, V = logits.shape
    t = []
    for j in range(R):
        best = 0
        for v in range(V):
            if logits[j, v] > logits[j, best]:
                best = v
        t.append(best)
    D = len(draft)
    a = max(a for a in range(D + 1) if all(draft[j] == t[j] for j in range(a)))
    bonus = t[a] if a < R else -1
    return a, bonus


def test_verify_greedy_brute_force_tiny_vocab():
    rng = np.random.default_rng(0)
    for _ in range(300):
        V = int(rng.integers(2, 5))
        D = int(rng.integers(1, 5))
        R = D + int(rng.integers(0, 2))
        lg = rng.integers(-2, 3, size=(1, R, V)).astype(np.float32)      # ties are common
        dr = rng.integers(0, V, size=(1, D))
        n_acc, bonus, committed = accept.verify_greedy(lg, dr)
        a, b = _brute_greedy(lg[0], list(dr[0]))
        assert (n_acc[0], bonus[0]) == (a, b)
        expect = list(dr[0][:a]) + ([b] if b >= 0 else [])
        expect += [-1] * (D + 1 - len(expect))
        assert list(committed[0]) == expect


def test_identical_P_and_Q_accept_the_whole_block():
    """Target logits equal to the drafter's logits: the argmax draft is fully accepted."""
    rng = np.random.default_rng(1)
    N, D, V = 3, 7, 50
    q_logits = rng.standard_normal((N, D + 1, V)).astype(np.float32)
    drafts = dnc.sample_drafts(q_logits[:, :D], 1, 0.0, 0)[:, 0]
    n_acc, bonus, committed = accept.verify_greedy(q_logits, drafts)
    assert np.all(n_acc == D)
    assert np.array_equal(bonus, q_logits[:, D].argmax(-1))
    assert np.array_equal(committed[:, :D], drafts)
    # only D rows: full accept, no bonus
    n_acc, bonus, committed = accept.verify_greedy(q_logits[:, :D], drafts)
    assert np.all(n_acc == D) and np.all(bonus == -1) and np.all(committed[:, D] == -1)


def test_planted_prefix_lengths_are_recovered():
    N, D, V = 16, 15, 300
    drafts = synth.make_drafts(N, 1, D, V, seed=4)[:, 0]
    logits, a = synth.make_planted_verify_logits(drafts, D + 1, V, 0.85, seed=4)
    n_acc, bonus, _ = accept.verify_greedy(logits.numpy(), drafts.numpy())
    assert np.array_equal(n_acc, a)
    assert np.all(bonus >= 0)


def test_alpha_tv_equals_sum_min():
    rng = np.random.default_rng(2)
    for V in (2, 5, 100):
        for _ in range(200):
            P = rng.dirichlet(np.ones(V))
            Q = rng.dirichlet(np.ones(V) * 0.3)
            assert abs(accept.alpha_tv(P, Q) - accept.alpha_min(P, Q)) < 1e-15


def test_alpha_one_hot_P_is_Q_of_target_token():
    """With a one-hot verifier the total-variation rate equals the probability that a draft
    sampled from Q hits the target's token (the greedy case)."""
    rng = np.random.default_rng(3)
    for V in (3, 10):
        Q = rng.dirichlet(np.ones(V))
        x = int(rng.integers(0, V))
        P = np.zeros(V)
        P[x] = 1.0
        assert abs(accept.alpha_tv(P, Q) - Q[x]) < 1e-15
        assert abs(accept.alpha_greedy_term(P, Q) - Q[x]) < 1e-15


def test_alpha_identical_P_Q_is_one():
    P = np.random.default_rng(4).dirichlet(np.ones(20))
    assert abs(accept.alpha_tv(P, P) - 1.0) < 1e-15


def test_alpha_monte_carlo_speculative_rule():
    rng = np.random.default_rng(5)
    V, n = 6, 200_000
    P = rng.dirichlet(np.ones(V))
    Q = rng.dirichlet(np.ones(V))
    a = accept.alpha_tv(P, Q)
    mc = accept.mc_speculative_accept_rate(P, Q, n, rng)
    assert abs(mc - a) < 4 * np.sqrt(a * (1 - a) / n)


def test_theorem_c3_lower_bound():
    """sum min(P, Q) >= sum P Q (min(a, b) >= ab on [0, 1])."""
    rng = np.random.default_rng(6)
    for _ in range(10_000):
        V = int(rng.integers(2, 30))
        P = rng.dirichlet(np.ones(V) * rng.uniform(0.1, 3))
        Q = rng.dirichlet(np.ones(V) * rng.uniform(0.1, 3))
        assert accept.alpha_min(P, Q) >= accept.alpha_greedy_term(P, Q) - 1e-15


def test_streak_expectation_matches_enumeration_and_monte_carlo():
    """Prefix-independent tiny case (V=4, gamma=3): the streak equation with per-position rates
    equals the exact expectation over every draft in V^gamma and a Monte Carlo estimate."""
    rng = np.random.default_rng(7)
    V, G = 4, 3
    P_rows = [rng.dirichlet(np.ones(V)) for _ in range(G)]
    Q_rows = [rng.dirichlet(np.ones(V)) for _ in range(G)]
    alphas = [accept.alpha_greedy_term(P_rows[j], Q_rows[j]) for j in range(G)]
    s = accept.streak_expectation(alphas)
    enum = accept.enum_streak_greedy(P_rows, Q_rows)
    assert abs(s - enum) < 1e-12
    n = 20_000
    mc = accept.mc_streak_greedy(P_rows, Q_rows, n, rng)
    # accepted length lies in [0, G]: the standard error is at most G / (2 sqrt(n))
    assert abs(mc - s) < 4 * G / (2 * np.sqrt(n))


def test_streak_score_by_hand():
    assert accept.streak_score([]) == 0.0
    assert accept.streak_score([1.0, 1.0, 1.0]) == 3.0
    assert accept.streak_score([0.5, 0.5]) == 0.5 + 0.25
    assert accept.streak_score([0.0, 1.0]) == 0.0


def test_argmax_draft_maximises_streak_score_brute_force():
    """S is increasing in each p_j, so the per-row argmax draft is the best draft in V^gamma."""
    rng = np.random.default_rng(8)
    for _ in range(30):
        V, G = int(rng.integers(2, 5)), int(rng.integers(1, 5))
        P_rows = [rng.dirichlet(np.ones(V)) for _ in range(G)]
        best, best_s = accept.brute_force_best_draft(P_rows)
        greedy = tuple(int(np.argmax(r)) for r in P_rows)
        assert abs(accept.streak_score([P_rows[j][x] for j, x in enumerate(greedy)]) - best_s) \
            < 1e-15


def test_select_streak_against_brute_force():
    """K drafts with prefix-dependent verifier rows: selection equals the brute-force maximiser
    of the exact-softmax streak score over the K candidates, and acceptance on it equals
    greedy verification of that draft alone."""
    rng = np.random.default_rng(9)
    for trial in range(40):
        N, K, G, V = 2, int(rng.integers(1, 6)), int(rng.integers(1, 5)), int(rng.integers(2, 7))
        R = G + int(rng.integers(0, 2))
        lg = (rng.standard_normal((N, K, R, V)) * 2).astype(np.float32)
        dr = rng.integers(0, V, size=(N, K, G))
        sel, scores, n_acc, bonus, committed = accept.select_streak(lg, dr)
        for n in range(N):
            exact = []
            for k in range(K):
                pr = accept.softmax64(lg[n, k])
                exact.append(accept.streak_score([pr[j, dr[n, k, j]] for j in range(G)]))
            exact = np.array(exact)
            # DNC scores within 1e-6 relative of the exact softmax scores
            assert np.all(np.abs(scores[n] - exact) <= 1e-6 * exact + 1e-12)
            top = np.sort(exact)[::-1]
            if K == 1 or top[0] - top[1] > 1e-5 * top[0]:
                assert sel[n] == int(np.argmax(exact))
            a, b, c = accept.verify_greedy(lg[n, sel[n]][None], dr[n, sel[n]][None])
            assert (n_acc[n], bonus[n]) == (a[0], b[0]) and np.array_equal(committed[n], c[0])


def test_select_streak_ties_go_to_lowest_k():
    V, G, K = 5, 3, 4
    row = np.zeros((G, V), np.float32)
    lg = np.broadcast_to(row, (1, K, G, V)).copy()
    dr = np.zeros((1, K, G), np.int64)
    sel, scores, *_ = accept.select_streak(lg, dr)
    assert sel[0] == 0 and np.all(scores[0] == scores[0, 0])


def test_select_streak_planted_streaks():
    N, K, G, V = 2, 4, 8, 200
    dr = synth.make_drafts(N, K, G, V, seed=3)
    lg, a = synth.make_planted_streak_logits(dr, G, V, 0.8, seed=3)
    sel, scores, n_acc, bonus, committed = accept.select_streak(lg.numpy(), dr.numpy())
    for n in range(N):
        assert n_acc[n] == a[n, sel[n]]
        if n_acc[n] == G:
            assert bonus[n] == -1          # only G rows: no bonus after a full accept


# ---- lossless stochastic verification (verify_sample) ----

def _broadcast(row, N):
    return np.broadcast_to(np.asarray(row, np.float32), (N,) + np.asarray(row).shape).copy()


def _spec_case(seed, V=8, t_p=1.0, t_q=1.0):
    rng = np.random.default_rng(seed)
    lp = (rng.normal(size=V) * 1.5).astype(np.float32)
    lq = (rng.normal(size=V) * 1.5).astype(np.float32)
    return lp, lq


def test_verify_sample_identical_P_and_Q_accept_everything():
    """P = Q: the ratio is 1 at every drafted token, so every position is accepted whatever the
    draw, and the bonus comes from row D."""
    rng = np.random.default_rng(3)
    N, D, V = 64, 5, 12
    dl = (rng.normal(size=(N, D, V)) * 2).astype(np.float32)
    tl = np.concatenate([dl, rng.normal(size=(N, 1, V)).astype(np.float32)], axis=1)
    drafts = dnc.sample_drafts(dl, 1, 1.0, seed=11)[:, 0]
    n_acc, bonus, committed = accept.verify_sample(tl, dl, drafts, 1.0, 1.0, seed=5)
    assert (n_acc == D).all()
    assert ((bonus >= 0) & (bonus < V)).all()
    assert (committed[:, :D] == drafts).all() and (committed[:, D] == bonus).all()
    # without a row D there is no bonus
    n_acc, bonus, committed = accept.verify_sample(dl, dl, drafts, 1.0, 1.0, seed=5)
    assert (n_acc == D).all() and (bonus == -1).all() and (committed[:, D] == -1).all()


def test_verify_sample_accept_rate_is_sum_min_monte_carlo():
    """Drafts x ~ Q (the DNC sampler), accepted with min(1, P/Q): the accept rate of one position
    is sum_x min(P(x), Q(x)) (SpecDiff-2 notes, section 5.1), checked against the fp64 softmax
    within 4 sigma."""
    N, V = 20_000, 8
    lp, lq = _spec_case(1, V)
    tl, dl = _broadcast(lp, N)[:, None], _broadcast(lq, N)[:, None]
    drafts = dnc.sample_drafts(dl, 1, 1.0, seed=21)[:, 0]
    n_acc, bonus, _ = accept.verify_sample(tl, dl, drafts, 1.0, 1.0, seed=22)
    a = accept.alpha_min(accept.softmax64(lp), accept.softmax64(lq))
    rate = float(np.mean(n_acc == 1))
    assert abs(rate - a) < 4 * np.sqrt(a * (1 - a) / N), (rate, a)


@pytest.mark.parametrize("t_p,t_q", [(1.0, 1.0), (1.0, 1.5), (0.7, 1.0)])
def test_verify_sample_output_is_distributed_as_P(t_p, t_q):
    """Losslessness: the committed token of a one-position block (the accepted draft or the
    replacement) is distributed as the target's P, whatever Q is: chi-square against the fp64
    softmax of the target row at its temperature."""
    from scipy import stats
    N, V = 20_000, 8
    lp, lq = _spec_case(2, V)
    tl, dl = _broadcast(lp, N)[:, None], _broadcast(lq, N)[:, None]
    drafts = dnc.sample_drafts(dl, 1, t_q, seed=31)[:, 0]
    _, _, committed = accept.verify_sample(tl, dl, drafts, t_p, t_q, seed=32)
    tok = committed[:, 0]
    assert (tok >= 0).all()
    P = accept.softmax64(lp, t_p)
    counts = np.bincount(tok, minlength=V)
    chi2 = float(((counts - N * P) ** 2 / (N * P)).sum())
    assert chi2 < stats.chi2.ppf(1 - 1e-4, V - 1), chi2


def test_verify_sample_second_position_and_bonus_are_distributed_as_P():
    """Two positions and a bonus row, all target rows independent of the prefix: whenever
    position 1 is committed it is distributed as P_1, and a bonus after a full accept as P_2."""
    from scipy import stats
    N, V = 30_000, 6
    rng = np.random.default_rng(4)
    lp = (rng.normal(size=(3, V)) * 1.2).astype(np.float32)
    lq = (rng.normal(size=(2, V)) * 1.2).astype(np.float32)
    tl, dl = _broadcast(lp, N), _broadcast(lq, N)
    drafts = dnc.sample_drafts(dl, 1, 1.0, seed=41)[:, 0]
    n_acc, bonus, committed = accept.verify_sample(tl, dl, drafts, 1.0, 1.0, seed=42)
    for pos, row in ((1, 1), (2, 2)):
        sel = n_acc >= pos
        tok = committed[sel, pos]
        P = accept.softmax64(lp[row])
        counts = np.bincount(tok, minlength=V)
        n = int(sel.sum())
        chi2 = float(((counts - n * P) ** 2 / (n * P)).sum())
        assert chi2 < stats.chi2.ppf(1 - 1e-4, V - 1), (pos, chi2)


def test_verify_sample_residual_mass_is_total_variation_exactly():
    """In integers, sum_v (qP_v ZQ - qQ_v ZP) = 0, so the residual mass W / (ZP ZQ) equals
    1 - sum_v min(P_v, Q_v) = (1/2) sum_v |P_v - Q_v| exactly (rational arithmetic)."""
    from fractions import Fraction
    rng = np.random.default_rng(6)
    for _ in range(20):
        V = int(rng.integers(2, 40))
        qP, ZP = dnc.row_weights((rng.normal(size=V) * 3).astype(np.float32))
        qQ, ZQ = dnc.row_weights((rng.normal(size=V) * 3).astype(np.float32), dnc.inv_temperature(1.5))
        diff = [int(a) * ZQ - int(b) * ZP for a, b in zip(qP, qQ)]
        assert sum(diff) == 0
        W = sum(accept.residual_weights(qP, ZP, qQ, ZQ))
        smin = sum(min(Fraction(int(a), ZP), Fraction(int(b), ZQ)) for a, b in zip(qP, qQ))
        tv = sum(abs(Fraction(int(a), ZP) - Fraction(int(b), ZQ)) for a, b in zip(qP, qQ)) / 2
        assert Fraction(W, ZP * ZQ) == 1 - smin == tv


def test_verify_sample_disjoint_supports_always_reject_and_resample_P():
    """Q's mass only on tokens where P is zero: every draft is rejected at position 0 and the
    replacement comes from P's support."""
    N, V = 500, 4
    lp = np.array([0.0, 0.3, -1e4, -1e4], np.float32)
    lq = np.array([-1e4, -1e4, 0.0, -0.2], np.float32)
    tl, dl = _broadcast(lp, N)[:, None], _broadcast(lq, N)[:, None]
    drafts = dnc.sample_drafts(dl, 1, 1.0, seed=51)[:, 0]
    assert set(drafts[:, 0].tolist()) <= {2, 3}
    n_acc, bonus, committed = accept.verify_sample(tl, dl, drafts, 1.0, 1.0, seed=52)
    assert (n_acc == 0).all()
    assert set(bonus.tolist()) == {0, 1}
    assert (committed[:, 0] == bonus).all() and (committed[:, 1] == -1).all()


def test_verify_sample_accept_test_by_hand():
    """u * qQ[x] * ZP < qP[x] * ZQ * 2^32 at its boundary, and out-of-vocabulary tokens."""
    qP, ZP = [1, 3], 4                      # P = (1/4, 3/4)
    qQ, ZQ = [1, 1], 2                      # Q = (1/2, 1/2): P(0)/Q(0) = 1/2
    half = 1 << 31
    assert accept.spec_accept_token(qP, ZP, qQ, ZQ, 0, half - 1)
    assert not accept.spec_accept_token(qP, ZP, qQ, ZQ, 0, half)
    assert accept.spec_accept_token(qP, ZP, qQ, ZQ, 1, (1 << 32) - 1)     # ratio 3/2 > 1
    assert not accept.spec_accept_token(qP, ZP, qQ, ZQ, 2, 0)
    assert not accept.spec_accept_token(qP, ZP, qQ, ZQ, -1, 0)
    # residual of P - Q = (-1/4, 1/4) is all on token 1
    assert accept.residual_weights(qP, ZP, qQ, ZQ) == [0, 2]      # 2 / (ZP ZQ) = 1/4
    assert accept.sample_from_weights([0, 4], 0) == 1
    assert accept.sample_from_weights([1, 1, 2], (1 << 32) - 1) == 2
    assert accept.sample_from_weights([1, 1, 2], 1 << 30) == 1      # thr = 1


def test_verify_sample_is_a_function_of_inputs_and_seed():
    rng = np.random.default_rng(7)
    N, D, V = 16, 4, 10
    tl = rng.normal(size=(N, D + 1, V)).astype(np.float32)
    dl = rng.normal(size=(N, D, V)).astype(np.float32)
    drafts = dnc.sample_drafts(dl, 1, 1.0, seed=3)[:, 0]
    a = accept.verify_sample(tl, dl, drafts, 1.0, 1.0, seed=9)
    b = accept.verify_sample(tl, dl, drafts, 1.0, 1.0, seed=9)
    c = accept.verify_sample(tl, dl, drafts, 1.0, 1.0, seed=10)
    assert all((x == y).all() for x, y in zip(a, b))
    assert any((x != y).any() for x, y in zip(a, c))
