"""Pins of the refinement oracle (Mask-Predict on the integer confidences)."""
import itertools

import numpy as np
import pytest

from oracle import dnc, refine


def _logits(rng, N, D, V, scale=2.0):
    """Random rows whose last token (the mask id in these tests) is never the argmax."""
    lg = (rng.standard_normal((N, D, V)) * scale).astype(np.float32)
    lg[..., -1] = -30.0
    return lg


def test_schedule_is_linear_from_all_to_none():
    assert [refine.remask_count(15, 3, t) for t in range(4)] == [15, 10, 5, 0]
    assert [refine.remask_count(16, 4, t) for t in range(5)] == [16, 12, 8, 4, 0]
    for D in (1, 7, 15, 64):
        for T in (1, 2, 3, 5, 10):
            n = [refine.remask_count(D, T, t) for t in range(T + 1)]
            assert n[0] == D and n[-1] == 0
            assert all(a >= b for a, b in zip(n, n[1:]))
            # the fraction masked falls by 1/T per pass, to within one position
            assert all(abs(n[t] - D * (T - t) / T) < 1 for t in range(T + 1))


def test_masked_positions_take_the_argmax_and_their_confidence():
    rng = np.random.default_rng(0)
    N, D, V = 2, 5, 300
    lg = _logits(rng, N, D, V)
    lg[0, 1, 7] = lg[0, 1, 9] = lg[0, 1].max() + 1.0          # planted tie: lowest index
    blk = np.full((N, D + 1), V - 1)
    blk[:, 0] = 3
    toks, cf = refine.refine_update(lg, blk, [[0] * D] * N, 0, 1, V - 1)
    assert np.array_equal(toks[:, 1:], np.argmax(lg, -1))
    assert toks[0, 2] == 7 and np.all(toks[:, 0] == 3)
    # 2^40 / Z is the largest softmax probability of the row (fp64), to the weights' accuracy
    for n in range(N):
        for j in range(D):
            x = lg[n, j].astype(np.float64)
            pmax = 1.0 / np.exp(x - x.max()).sum()
            assert abs((2.0 ** 40 / cf[n][j]) / pmax - 1) < 1e-5


def test_kept_positions_are_not_touched():
    rng = np.random.default_rng(1)
    N, D, V = 1, 6, 50
    lg = _logits(rng, N, D, V)
    blk = np.array([[11, 20, 21, 49, 23, 49, 25]])
    conf = [[5, 6, 0, 7, 0, 8]]
    toks, cf = refine.refine_update(lg, blk, conf, 0, 1, 49)
    for j in (0, 1, 3, 5):
        assert toks[0, 1 + j] == blk[0, 1 + j] and cf[0][j] == conf[0][j]
    for j in (2, 4):
        assert toks[0, 1 + j] == np.argmax(lg[0, j]) and cf[0][j] == dnc.row_weights(lg[0, j])[1]


@pytest.mark.parametrize("n_remask", [0, 1, 2, 3, 5, 6])
def test_remasked_set_is_the_unique_least_confident_one(n_remask):
    """Brute force over every subset: the remasked positions are the only set of that size whose
    every member is less confident than every kept position (larger Z, lower index on ties)."""
    rng = np.random.default_rng(n_remask)
    D, V = 6, 40
    lg = _logits(rng, 1, D, V)
    lg[0, 4] = lg[0, 1]                       # equal rows: equal Z, the tie rule decides
    lg[0, 5] = lg[0, 1]
    toks, cf = refine.refine_update(lg, np.full((1, D), V - 1), [[0] * D], n_remask, 0, V - 1)
    Z = [dnc.row_weights(lg[0, j])[1] for j in range(D)]
    assert Z[1] == Z[4] == Z[5]

    def below(j, k):                          # j is less confident than k
        return Z[j] > Z[k] or (Z[j] == Z[k] and j < k)

    ok = [set(S) for S in itertools.combinations(range(D), n_remask)
          if all(below(j, k) for j in S for k in range(D) if k not in S)]
    assert len(ok) == 1
    got = {j for j in range(D) if toks[0, j] == V - 1}
    assert got == ok[0]
    assert all((cf[0][j] == 0) == (j in got) for j in range(D))


def test_one_pass_is_the_argmax_draft():
    rng = np.random.default_rng(2)
    N, D, V = 3, 7, 100
    lg = _logits(rng, N, D, V)
    blk = np.full((N, D + 1), V - 1)
    blk[:, 0] = 5
    final, fed = refine.mask_predict(lambda b: lg, blk, 1, V - 1, 1)
    assert len(fed) == 1 and np.array_equal(fed[0], blk)
    assert np.array_equal(final[:, 1:], np.argmax(lg, -1))


def test_block_independent_forward_is_a_fixed_point():
    """When the forward ignores the block, every pass re-drafts the same tokens; the fed blocks
    carry the scheduled number of masks."""
    rng = np.random.default_rng(3)
    N, D, V, T = 2, 9, 64, 4
    lg = _logits(rng, N, D, V)
    blk = np.full((N, D), V - 1)
    final, fed = refine.mask_predict(lambda b: lg, blk, 0, V - 1, T)
    assert np.array_equal(final, np.argmax(lg, -1))
    for t, b in enumerate(fed):
        assert np.all((b == V - 1).sum(1) == refine.remask_count(D, T, t))


def test_block_dependent_forward_keeps_confident_tokens():
    """A forward whose preferred token at j is (j + number of visible tokens) mod V: tokens kept
    between passes never change, re-masked ones are re-drafted from the new block."""
    N, D, V, T = 1, 8, 32, 3
    mask = V - 1
    rng = np.random.default_rng(4)
    noise = _logits(rng, N, D, V, 0.1)

    def fwd(b):
        vis = int((b[0] != mask).sum())
        lg = noise.copy()
        for j in range(D):
            lg[0, j, (j + vis) % (V - 1)] += 3.0 + 0.2 * j
        return lg

    final, fed = refine.mask_predict(fwd, np.full((N, D), mask), 0, mask, T)
    for a, b in zip(fed[1:], fed[2:] + [final]):
        kept = a[0] != mask
        assert np.array_equal(a[0][kept], b[0][kept])
    last = fwd(fed[-1])
    remasked = fed[-1][0] == mask
    assert np.array_equal(final[0][remasked], np.argmax(last[0], -1)[remasked])
    assert not np.any(final == mask)
