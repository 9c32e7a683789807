"""verify_greedy_noalloc, the entry point for callers that cannot allocate (its partials live in
the library's static device scratch), against verify_greedy with a caller workspace: identical
outputs on two calls in a row, the second smaller, so a stale first call's scratch is never
read; and against the oracle."""
import numpy as np
import pytest
import torch

import block_diffusion_drafter_draft_amd as dbd
import synth
from oracle import accept

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _outputs(N, D):
    return (torch.full((N,), -7, dtype=torch.int32, device=DEV),
            torch.full((N,), -7, dtype=torch.int32, device=DEV),
            torch.full((N, D + 1), -7, dtype=torch.int32, device=DEV),
            torch.full((N,), -7, dtype=torch.int32, device=DEV))


def _both(N, D, R, V, seed):
    print(f"verify_greedy_noalloc N={N} D={D} R={R} V={V}", flush=True)
    drafts = synth.make_drafts(N, 1, D, V, seed=seed, device=DEV)[:, 0].contiguous()
    logits, planted = synth.make_planted_verify_logits(drafts, R, V, 0.85, seed=seed, device=DEV)
    got = []
    for noalloc in (False, True):
        na, bo, com, fl = _outputs(N, D)
        if noalloc:
            dbd.verify_greedy_noalloc(logits, drafts, na, bo, com, row_flags=fl)
        else:
            ws = torch.empty(dbd.verify_workspace_bytes(N, R, V), dtype=torch.uint8, device=DEV)
            dbd.verify_greedy(logits, drafts, na, bo, com, ws, row_flags=fl)
        torch.cuda.synchronize()
        got.append([t.cpu().numpy() for t in (na, bo, com, fl)])
    for a, b in zip(got[1], got[0]):
        assert np.array_equal(a, b)
    ref = accept.verify_greedy(logits.cpu().numpy(), drafts.cpu().numpy())
    for a, b in zip(got[1][:3], ref):
        assert np.array_equal(a, b)
    assert np.array_equal(got[1][0], planted) and np.all(got[1][3] == 0)


def test_noalloc_verify_equals_workspace_verify_on_two_calls():
    _both(32, 15, 16, 151936, seed=21)       # the Qwen3-8B-shaped batch: 512 rows
    _both(3, 7, 8, 4099, seed=22)            # smaller, ragged vocab, bonus row present
