"""Deterministic numerics contract (DNC): the slow, plain CPU definition.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this package; only the tests,
the smoke check and the bench's CPU-baseline leg do.

The pages fix what is computed but not how to make a sampled token or a selected draft a pure
function of the logits.  SpecDiff-2 notes, section 5.2: K joint drafts are drawn independently
from the single-step marginals at a temperature, and the draft with the largest streak score is
picked from the verifier's per-token posteriors.  To make those integer results identical on any
hardware, probabilities are built from integers:

  R1  argmax: the lowest index among the maxima.
  R2  exp_dnc(x), x <= 0, all in fp32 with every multiply and add rounded separately:
      Cody-Waite range reduction (Cody & Waite, 1980) by ln 2 split in a high part with 16
      significant bits and a low part, then the degree-7 Taylor polynomial of e^r in Horner form,
      then scaling by 2^k.  Arguments with x*log2(e) < -64 give 0.
  R3  integer weights of a row: M = row max (fp32); e_v = exp_dnc((l_v - M) * invT) in fp32;
      q_v = floor(e_v * 2^40); Z = sum q_v exactly (an integer, order free).
  R4  counter RNG: the SplitMix64 finaliser (Steele, Lea & Flood, OOPSLA 2014); the draw for
      (n, k, j) is u = mix64(mix64(seed) + (idx + 1) * 0x9E3779B97F4A7C15) >> 32 with
      idx = (n*K + k)*D + j, all modulo 2^64.
  R5  sampling: thr = (u * Z) >> 32; token = the smallest v with q_0 + ... + q_v > thr.
  R6  selection probability of token x: double(q_x) / double(Z), each rounded to nearest.
  Top-p (a reading; the pages name no nucleus rule): the nucleus is the shortest run of tokens,
      in order of decreasing weight with ties by increasing index, whose mass reaches
      ceil(p * Z) for p the float32 value (a dyadic rational, so the ceiling is exact); the draw
      is R5 on the weights restricted to it.
"""
import math

import numpy as np

_F = np.float32
_M64 = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15          # 2^64 / golden ratio, the SplitMix64 increment
FRAC_BITS = 40                       # R3 fixed-point scale


def _f32(x) -> np.float32:
    return np.float32(x)


# R2 constants, each derived from its mathematical definition.
LOG2E = _f32(1.0 / math.log(2.0))
# ln 2 rounded to fp32, then its 8 lowest mantissa bits cleared: 16 significant bits, so that
# k * LN2_HI is exact for |k| <= 128.
LN2_HI = np.frombuffer((np.frombuffer(_f32(math.log(2.0)).tobytes(), np.uint32)
                        & np.uint32(0xFFFFFF00)).tobytes(), np.float32)[0]
LN2_LO = _f32(math.log(2.0) - float(LN2_HI))
TAYLOR = [_f32(1.0 / math.factorial(i)) for i in range(8)]   # c0 .. c7


def exp_dnc(x) -> np.ndarray:
    """R2 on an fp32 array of arguments <= 0; returns fp32."""
    x = np.asarray(x, dtype=np.float32)
    t = (x * LOG2E).astype(np.float32)
    k = np.rint(t).astype(np.float32)                  # round half to even
    r = (x - (k * LN2_HI).astype(np.float32)).astype(np.float32)
    r = (r - (k * LN2_LO).astype(np.float32)).astype(np.float32)
    p = np.full_like(r, TAYLOR[7])
    for c in TAYLOR[6::-1]:
        p = (p * r).astype(np.float32)
        p = (p + c).astype(np.float32)
    out = np.ldexp(p, k.astype(np.int32)).astype(np.float32)
    return np.where(t < _f32(-64.0), _f32(0.0), out).astype(np.float32)


def inv_temperature(temperature: float) -> np.float32:
    """fp32 of 1/T, the reciprocal taken in fp64."""
    return _f32(1.0 / float(temperature))


def row_weights(row, inv_t=np.float32(1.0)):
    """R3 for one fp32 row: (q as a uint64 numpy array, Z as a Python int)."""
    row = np.asarray(row, dtype=np.float32)
    m = row[argmax_lowest(row)]
    z = ((row - m).astype(np.float32) * _f32(inv_t)).astype(np.float32)
    e = exp_dnc(z)
    scaled = (e.astype(np.float64) * float(1 << FRAC_BITS))     # exact: e * 2^40 fits in fp64
    q = np.floor(scaled).astype(np.uint64)
    Z = int(q.sum(dtype=np.uint64))      # exact: V * 2^40 < 2^64
    return q, Z


def argmax_lowest(row) -> int:
    """R1: index of the first occurrence of the maximum (IEEE compare, so +0 == -0).
    numpy's argmax returns the first occurrence; the tests pin this on planted ties."""
    return int(np.argmax(np.asarray(row)))


def mix64(z: int) -> int:
    """SplitMix64 output function on a 64-bit integer."""
    z &= _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def draw_u32(seed: int, n: int, k: int, j: int, n_drafts: int, n_pos: int) -> int:
    """R4: the 32-bit uniform draw for sequence n, draft k, position j."""
    idx = (n * n_drafts + k) * n_pos + j
    return mix64((mix64(seed) + (idx + 1) * GOLDEN) & _M64) >> 32


def sample_token(q, Z: int, u: int) -> int:
    """R5: first index whose inclusive prefix sum of q exceeds (u * Z) >> 32."""
    thr = (int(u) * int(Z)) >> 32
    prefix = np.cumsum(q, dtype=np.uint64)          # exact integer prefix sums
    v = int(np.searchsorted(prefix, np.uint64(thr), side="right"))
    assert v < prefix.shape[0], "threshold beyond total mass"
    return v


def top_p_threshold(Z: int, top_p: float) -> int:
    """ceil(p * Z) for p the float32 value of top_p, exactly (p is a dyadic rational)."""
    from fractions import Fraction
    return math.ceil(Fraction(float(np.float32(top_p))) * int(Z))


def nucleus_weights(q, Z: int, top_p: float):
    """Top-p filter on integer weights: the tokens ordered by weight (descending), ties by index
    (ascending); the nucleus is the shortest prefix of that order whose mass reaches
    ceil(p * Z); weights outside it become 0.  p >= 1 keeps every token."""
    q = [int(a) for a in q]
    if float(np.float32(top_p)) >= 1.0:
        return q
    need = top_p_threshold(Z, top_p)
    order = sorted(range(len(q)), key=lambda v: (-q[v], v))
    keep, mass = set(), 0
    for v in order:
        if mass >= need:
            break
        keep.add(v)
        mass += q[v]
    return [a if v in keep else 0 for v, a in enumerate(q)]


def sample_drafts(logits, n_drafts: int, temperature: float, seed: int,
                  top_p: float = 1.0) -> np.ndarray:
    """K joint drafts per sequence from single-step marginals (SpecDiff-2 notes, section 5.2).

    logits: [N, D, V] fp32.  temperature <= 0 gives the argmax draft (K must be 1).  top_p < 1
    restricts each position's draw to its nucleus (``nucleus_weights``); the draw is R5 on the
    restricted weights, in token order.
    Returns [N, K, D] int32."""
    logits = np.asarray(logits, dtype=np.float32)
    N, D, V = logits.shape
    out = np.zeros((N, n_drafts, D), dtype=np.int32)
    if temperature <= 0:
        assert n_drafts == 1
        for n in range(N):
            for j in range(D):
                out[n, 0, j] = argmax_lowest(logits[n, j])
        return out
    inv_t = inv_temperature(temperature)
    for n in range(N):
        for j in range(D):
            q, Z = row_weights(logits[n, j], inv_t)
            if float(np.float32(top_p)) < 1.0:
                w = nucleus_weights(q, Z, top_p)
                q, Z = np.array(w, dtype=np.uint64), sum(w)
            for k in range(n_drafts):
                out[n, k, j] = sample_token(q, Z, draw_u32(seed, n, k, j, n_drafts, D))
    return out


def token_prob(row, token: int, inv_t=np.float32(1.0)) -> float:
    """R6: DNC probability of ``token`` under one fp32 logit row."""
    q, Z = row_weights(row, inv_t)
    return float(int(q[token])) / float(Z)
