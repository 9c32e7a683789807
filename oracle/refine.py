"""Iterative refinement of a drafted block.

TEST INFRASTRUCTURE: part of the CPU oracle (see the package docstring); only the tests, the
smoke check and the bench's CPU-baseline leg may import it.

The DFlash article (its section on writing a whole block in one forward pass) says the drafter
emits the block in one forward pass and refines it when needed; no page states how.  Reading:
Mask-Predict (Ghazvininejad, Levy, Liu and Zettlemoyer, EMNLP 2019), the published rule for
refining parallel masked predictions.  A block of D drafted positions gets T forward passes; the
first drafts every position; before pass t (1 <= t < T) the n_t = floor(D (T - t) / T) least
confident positions are masked again and re-drafted by the next pass, while the others keep their
tokens and confidences.

Confidence of a drafted position: the probability of its argmax token at temperature 1 under the
library's integer weights (``dnc.row_weights``).  The argmax token's weight is always 2^40, so the
probability is 2^40 / Z and orders exactly like 1 / Z: the least confident position is the one
with the largest Z, and among equal Z the lower position index goes first.
"""
import numpy as np

from . import dnc


def remask_count(n_draft: int, n_passes: int, t: int) -> int:
    """Mask-Predict's linear schedule: positions masked before pass t of n_passes (t = 0: all)."""
    return (n_draft * (n_passes - t)) // n_passes


def refine_update(logits, block_tokens, conf, n_remask: int, n_anchor: int, mask_id: int):
    """One refinement update of a batch after a forward pass.

    logits [N, D, V] fp32: the forward's LM-head rows of the D drafted positions;
    block_tokens [N, B]: the block that forward read (anchor first when n_anchor = 1);
    conf [N, D] (Python ints): 0 marks a position that was masked in that forward, otherwise the
    position's Z from the pass that drafted it;
    n_remask: positions to mask again for the next pass (0 after the last pass).

    Masked positions take the argmax token of their row and its Z as confidence; then the
    n_remask positions of largest Z (lower index first on ties) become mask_id with conf 0.
    Returns (block_tokens', conf') as (int64 array [N, B], list of lists of ints)."""
    logits = np.asarray(logits, dtype=np.float32)
    N, D, _ = logits.shape
    toks = np.array(block_tokens, dtype=np.int64).copy()
    cf = [[int(c) for c in row] for row in conf]
    for n in range(N):
        for j in range(D):
            if cf[n][j] == 0:
                row = logits[n, j]
                toks[n, n_anchor + j] = dnc.argmax_lowest(row)
                cf[n][j] = dnc.row_weights(row)[1]
        order = sorted(range(D), key=lambda j: (-cf[n][j], j))
        for j in order[:n_remask]:
            toks[n, n_anchor + j] = mask_id
            cf[n][j] = 0
    return toks, cf


def mask_predict(forward, block_tokens, n_anchor: int, mask_id: int, n_passes: int):
    """T = n_passes forward passes of Mask-Predict from a block whose D positions are all masked.

    forward(block [N, B] int64) -> logits [N, D, V].  Returns (the final block, the list of the
    blocks fed to the passes)."""
    blk = np.array(block_tokens, dtype=np.int64)
    N, B = blk.shape
    D = B - n_anchor
    conf = [[0] * D for _ in range(N)]
    fed = []
    for t in range(n_passes):
        fed.append(blk.copy())
        blk, conf = refine_update(forward(blk), blk, conf, remask_count(D, n_passes, t + 1),
                                  n_anchor, mask_id)
    return blk, fed
