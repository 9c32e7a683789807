"""Verify/accept step: the slow, plain CPU definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* Greedy verification (DFlare page, section on drafting in parallel and accepting with the
  target): the target checks the block; under greedy decoding the prefix up to the first mismatch
  is kept and the target's own next token is appended.
* Self-selection (SpecDiff-2 notes, section 5.2): among K joint drafts, the one with the largest
  expected streak sum_m prod_{j<=m} p_j under the verifier's per-token posteriors is chosen, then
  greedy acceptance runs on it, reusing the cached verifier outputs.
* Streak equation and acceptance rate (SpecDiff-2 notes, section 5.1): the expected accepted
  tokens per draft is E[sum_m prod_{j<=m} alpha_j]; alpha = 1 - (1/2)||P - Q||_1.
* Lossless stochastic verification (SpecDiff-2 notes, sections 4 and 5.1): the
  speculative-sampling rule on the integer weights, ``verify_sample``.

Readings where the pages are silent (each listed with its reason in the design notes):
* target row j scores the token at draft position j; with D+1 rows the last one gives the bonus
  after a full accept, with only D rows a full accept has no bonus (-1);
* ties go to the lowest token index and to the lowest draft index;
* the verifier posterior for the streak score is the temperature-1 softmax of the given logits,
  computed through the integer weights of ``dnc``.
"""
import itertools

import numpy as np

from . import dnc


def greedy_accept_row_tokens(target_tokens, draft, n_rows: int):
    """Greedy acceptance from the target's per-row argmax tokens.

    target_tokens: length-R sequence (t_j = argmax of target row j); draft: length-D tokens.
    Returns (n_acc, bonus, committed) with committed of length D+1, padded with -1."""
    D = len(draft)
    n_acc = 0
    while n_acc < D and int(draft[n_acc]) == int(target_tokens[n_acc]):
        n_acc += 1
    bonus = int(target_tokens[n_acc]) if n_acc < n_rows else -1
    committed = [int(t) for t in draft[:n_acc]]
    if bonus >= 0:
        committed.append(bonus)
    committed += [-1] * (D + 1 - len(committed))
    return n_acc, bonus, committed


def verify_greedy(target_logits, drafts):
    """target_logits: [N, R, V] fp32 with R in {D, D+1}; drafts: [N, D] ints.
    Returns (n_accepted [N], bonus [N], committed [N, D+1]) as int32 arrays."""
    target_logits = np.asarray(target_logits, dtype=np.float32)
    drafts = np.asarray(drafts)
    N, R, V = target_logits.shape
    D = drafts.shape[1]
    assert R in (D, D + 1)
    n_acc = np.zeros(N, np.int32)
    bonus = np.zeros(N, np.int32)
    committed = np.zeros((N, D + 1), np.int32)
    for n in range(N):
        t = [dnc.argmax_lowest(target_logits[n, j]) for j in range(R)]
        a, b, c = greedy_accept_row_tokens(t, drafts[n], R)
        n_acc[n], bonus[n], committed[n] = a, b, c
    return n_acc, bonus, committed


def streak_score(probs) -> float:
    """sum_{m=1..G} prod_{j<=m} p_j, in fp64 and in position order (P = P*p_j; S = S + P)."""
    P = 1.0
    S = 0.0
    for p in probs:
        P = P * float(p)
        S = S + P
    return S


def select_streak(verifier_logits, drafts):
    """verifier_logits: [N, K, R, V] fp32, R in {G, G+1}; drafts: [N, K, G].

    Row (n, k, j) is the verifier's distribution for position j of draft k given that draft's
    prefix.  Returns (selected [N], scores [N, K] fp64, n_accepted [N], bonus [N],
    committed [N, G+1])."""
    verifier_logits = np.asarray(verifier_logits, dtype=np.float32)
    drafts = np.asarray(drafts)
    N, K, R, V = verifier_logits.shape
    G = drafts.shape[2]
    assert R in (G, G + 1)
    selected = np.zeros(N, np.int32)
    scores = np.zeros((N, K), np.float64)
    n_acc = np.zeros(N, np.int32)
    bonus = np.zeros(N, np.int32)
    committed = np.zeros((N, G + 1), np.int32)
    for n in range(N):
        best = 0
        for k in range(K):
            p = [dnc.token_prob(verifier_logits[n, k, j], int(drafts[n, k, j]))
                 for j in range(G)]
            scores[n, k] = streak_score(p)
            if scores[n, k] > scores[n, best]:
                best = k
        selected[n] = best
        t = [dnc.argmax_lowest(verifier_logits[n, best, j]) for j in range(R)]
        a, b, c = greedy_accept_row_tokens(t, drafts[n, best], R)
        n_acc[n], bonus[n], committed[n] = a, b, c
    return selected, scores, n_acc, bonus, committed


def spec_accept_token(qP, ZP: int, qQ, ZQ: int, x: int, u: int) -> bool:
    """Accept draft token x with probability min(1, P(x)/Q(x)), P(x) = qP[x]/ZP, Q(x) = qQ[x]/ZQ,
    for a uniform 32-bit draw u: accepted iff u/2^32 < P(x)/Q(x), i.e. in integers
    u * qQ[x] * ZP < qP[x] * ZQ * 2^32.  A token outside the vocabulary has P = Q = 0 and is
    rejected."""
    V = len(qP)
    px = int(qP[x]) if 0 <= x < V else 0
    qx = int(qQ[x]) if 0 <= x < V else 0
    return int(u) * qx * int(ZP) < px * int(ZQ) * (1 << 32)


def residual_weights(qP, ZP: int, qQ, ZQ: int):
    """Integer weights of norm(max(0, P - Q)): w_v = max(0, qP[v]*ZQ - qQ[v]*ZP), a common
    multiple ZP*ZQ of P - Q (Python ints, exact)."""
    return [max(0, int(a) * int(ZQ) - int(b) * int(ZP)) for a, b in zip(qP, qQ)]


def sample_from_weights(w, u: int) -> int:
    """R5 on arbitrary non-negative integer weights: the first v whose inclusive prefix sum
    exceeds (u * W) >> 32, W = sum(w)."""
    W = sum(int(a) for a in w)
    thr = (int(u) * W) >> 32
    run = 0
    for v, a in enumerate(w):
        run += int(a)
        if run > thr:
            return v
    raise AssertionError("threshold beyond total mass")


def verify_sample(target_logits, draft_logits, drafts, t_target: float, t_draft: float,
                  seed: int):
    """Lossless stochastic verification of one draft per sequence (SpecDiff-2 notes, section 4:
    the verifier applies a lossless acceptance rule left to right; section 5.1: its accept rate
    alpha_SD = sum_x min(P, Q)).  The rule is the speculative-sampling rule (Leviathan et al.,
    2023), on the integer weights of ``dnc``:

    for j = 0 .. D-1: P_j from target row j at t_target, Q_j from draft row j at t_draft; accept
    x_j with probability min(1, P_j(x_j)/Q_j(x_j)) (draw (n, 0, j)).  At the first rejection the
    replacement token is drawn (draw (n, 1, j)) from norm(max(0, P_j - Q_j)), or from P_j when
    that is zero everywhere; the drafts before it and the replacement are committed.  If every
    position is accepted and a target row D exists, a bonus token is drawn from P_D (draw
    (n, 1, D)); with only D rows there is no bonus (-1).  Draws are R4 with K = 2 streams over
    D + 1 positions.

    target_logits [N, R, V] fp32 (R = D or D+1); draft_logits [N, D, V] fp32 (the drafter's
    logits the drafts were sampled from); drafts [N, D] int.
    Returns (n_acc [N], bonus [N], committed [N, D+1] padded with -1)."""
    target_logits = np.asarray(target_logits, dtype=np.float32)
    draft_logits = np.asarray(draft_logits, dtype=np.float32)
    drafts = np.asarray(drafts)
    N, R, V = target_logits.shape
    D = drafts.shape[1]
    assert R in (D, D + 1) and draft_logits.shape == (N, D, V)
    inv_p = dnc.inv_temperature(t_target)
    inv_q = dnc.inv_temperature(t_draft)
    n_acc = np.zeros(N, np.int32)
    bonus = np.full(N, -1, np.int32)
    committed = np.full((N, D + 1), -1, np.int32)
    for n in range(N):
        a, b = D, -1
        for j in range(D):
            qP, ZP = dnc.row_weights(target_logits[n, j], inv_p)
            qQ, ZQ = dnc.row_weights(draft_logits[n, j], inv_q)
            x = int(drafts[n, j])
            u = dnc.draw_u32(seed, n, 0, j, 2, D + 1)
            if spec_accept_token(qP, ZP, qQ, ZQ, x, u):
                continue
            w = residual_weights(qP, ZP, qQ, ZQ)
            if sum(w) == 0:
                w = [int(c) for c in qP]
            a, b = j, sample_from_weights(w, dnc.draw_u32(seed, n, 1, j, 2, D + 1))
            break
        else:
            if R > D:
                qP, ZP = dnc.row_weights(target_logits[n, D], inv_p)
                b = sample_from_weights([int(c) for c in qP], dnc.draw_u32(seed, n, 1, D, 2, D + 1))
        n_acc[n], bonus[n] = a, b
        committed[n, :a] = drafts[n, :a]
        if b >= 0:
            committed[n, a] = b
    return n_acc, bonus, committed


# ---- helpers for the self-checks (SpecDiff-2 notes, section 5.1) ----

def softmax64(logits, temperature: float = 1.0):
    z = np.asarray(logits, dtype=np.float64) / float(temperature)
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def alpha_tv(P, Q) -> float:
    """1 - (1/2) sum_x |P(x) - Q(x)|."""
    return 1.0 - 0.5 * float(np.abs(np.asarray(P, np.float64) - np.asarray(Q, np.float64)).sum())


def alpha_min(P, Q) -> float:
    """sum_x min(P(x), Q(x)): accept rate of the speculative-sampling rule."""
    return float(np.minimum(np.asarray(P, np.float64), np.asarray(Q, np.float64)).sum())


def alpha_greedy_term(P, Q) -> float:
    """E_{x~P}[Q(x)] = sum_x P(x) Q(x): the per-position term of the streak-distillation
    objective."""
    return float((np.asarray(P, np.float64) * np.asarray(Q, np.float64)).sum())


def streak_expectation(alphas) -> float:
    """Streak equation with per-position rates: sum_m prod_{j<=m} alpha_j."""
    return streak_score(alphas)


def mc_speculative_accept_rate(P, Q, n_trials: int, rng) -> float:
    """Monte Carlo of the speculative-sampling rule: draw x ~ Q, accept with min(1, P(x)/Q(x))."""
    P = np.asarray(P, np.float64)
    Q = np.asarray(Q, np.float64)
    x = rng.choice(len(Q), size=n_trials, p=Q)
    u = rng.random(n_trials)
    ratio = np.where(Q[x] > 0, P[x] / np.where(Q[x] > 0, Q[x], 1.0), 0.0)
    return float(np.mean(u < np.minimum(1.0, ratio)))


def mc_streak_greedy(P_rows, Q_rows, n_trials: int, rng) -> float:
    """Monte Carlo of accepted tokens per draft when the draft is sampled position by position
    from Q_rows and each position is checked against a sample from the verifier's P_rows (a
    prefix-independent verifier): count leading positions where the two samples agree."""
    G = len(P_rows)
    total = 0
    for _ in range(n_trials):
        m = 0
        while m < G:
            x = rng.choice(len(Q_rows[m]), p=Q_rows[m])
            y = rng.choice(len(P_rows[m]), p=P_rows[m])
            if x != y:
                break
            m += 1
        total += m
    return total / n_trials


def enum_streak_greedy(P_rows, Q_rows) -> float:
    """Exact expectation of the same quantity by enumerating every draft in V^G and every verifier
    sample sequence, weighting each by its probability (tiny V and G only)."""
    G = len(P_rows)
    V = len(P_rows[0])
    total = 0.0
    for xs in itertools.product(range(V), repeat=G):
        pq = 1.0
        for j, x in enumerate(xs):
            pq *= Q_rows[j][x]
        if pq == 0.0:
            continue
        # accepted length distribution given the draft: position j accepted w.p. P_rows[j][x_j]
        acc = 0.0
        run = 1.0
        for j, x in enumerate(xs):
            run *= P_rows[j][x]
            acc += run
        total += pq * acc
    return total


def brute_force_best_draft(P_rows):
    """The draft in V^G maximising sum_m prod_{j<=m} P_rows[j][x_j] (ties: lexicographically
    smallest), by enumeration."""
    G = len(P_rows)
    V = len(P_rows[0])
    best, best_s = None, -1.0
    for xs in itertools.product(range(V), repeat=G):
        s = streak_score([P_rows[j][x] for j, x in enumerate(xs)])
        if s > best_s:
            best, best_s = xs, s
    return best, best_s
