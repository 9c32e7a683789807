"""Block refinement (Mask-Predict reading) on the GPU against the oracle: the update alone,
bit-exact, and whole refinement loops of draft_block passes."""
import numpy as np
import pytest
import torch

import block_diffusion_drafter_draft_amd as dbd
import synth
from oracle import dnc
from oracle import drafter as od
from oracle import refine
from drafter_case import Case, rel_l2

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = {"f32": 1e-4, "bf16": 2e-2}


def _refine_gpu(lg, blk, conf, n_anchor, mask_id, n_remask):
    N, D, V = lg.shape
    ws = torch.empty(dbd.refine_workspace_bytes(N, D, V), dtype=torch.uint8, device=DEV)
    b, c = blk.clone(), conf.clone()
    dbd.refine_block(lg, b, c, n_anchor, mask_id, n_remask, ws)
    torch.cuda.synchronize()
    return b, c


def _check_update(lg, blk, conf, n_anchor, mask_id, n_remask):
    b, c = _refine_gpu(lg, blk, conf, n_anchor, mask_id, n_remask)
    rb, rc = refine.refine_update(lg.cpu().numpy(), blk.cpu().numpy(),
                                  [[int(x) for x in row] for row in conf.cpu().numpy()],
                                  n_remask, n_anchor, mask_id)
    assert np.array_equal(b.cpu().numpy(), rb)
    assert [[int(x) for x in row] for row in c.cpu().numpy()] == rc
    return b, c


@pytest.mark.parametrize("N,B,n_anchor,V,n_remask", [
    (3, 16, 1, 4099, 0), (3, 16, 1, 4099, 7), (3, 16, 1, 4099, 15), (2, 64, 0, 1000, 33),
    (4, 8, 1, 151936, 2), (1, 2, 1, 50, 1), (2, 64, 0, 3, 63)])
def test_refine_update_bit_exact(N, B, n_anchor, V, n_remask):
    """Mixed states (positions to fill next to kept ones), equal rows and a kept confidence equal
    to a fresh Z, so the index tie rule decides."""
    print(f"refine N={N} B={B} anchor={n_anchor} V={V} n_remask={n_remask}", flush=True)
    D = B - n_anchor
    g = torch.Generator(device=DEV).manual_seed(N * 7 + B + V)
    lg = torch.randn((N, D, V), generator=g, device=DEV) * 2.0
    if D >= 6:
        lg[0, 3] = lg[0, 1]
        lg[0, 5] = lg[0, 1]
    rng = np.random.default_rng(B + V)
    conf = np.where(rng.random((N, D)) < 0.5, 0,
                    rng.integers(1 << 40, 1 << 52, (N, D))).astype(np.int64)
    if D >= 6:
        conf[0, 1] = conf[0, 3] = 0
        conf[0, 4] = dnc.row_weights(lg[0, 1].cpu().numpy())[1]
    blk = torch.from_numpy(rng.integers(0, V - 1, (N, B)).astype(np.int32)).to(DEV)
    blk[:, n_anchor:][torch.from_numpy(conf == 0).to(DEV)] = V - 1
    _check_update(lg, blk, torch.from_numpy(conf).to(DEV), n_anchor, V - 1, n_remask)


def test_refine_all_masked_then_final():
    """From an all-masked block: the update with n_remask = 0 is the argmax draft."""
    N, B, V = 3, 12, 2000
    g = torch.Generator(device=DEV).manual_seed(5)
    lg = torch.randn((N, B - 1, V), generator=g, device=DEV) * 3.0
    blk = torch.full((N, B), V - 1, dtype=torch.int32, device=DEV)
    blk[:, 0] = 17
    conf = torch.zeros((N, B - 1), dtype=torch.int64, device=DEV)
    b, c = _check_update(lg, blk, conf, 1, V - 1, 0)
    assert torch.equal(b[:, 1:].long(), lg.argmax(-1)) and torch.all(b[:, 0] == 17)
    assert torch.all(c > 0)


def _loop(wl, n_passes, seqs=None):
    """n_passes draft_block passes with refine_block between them; every pass's logits against
    the oracle forward on the same block, every update bit-exact against the oracle's."""
    sh = wl.shape
    case = Case(wl, dev=DEV)
    case.fill_cache()
    N, D, mask = wl.batch, case.D, sh.mask_token_id
    blk = case.tokens.clone()
    conf = torch.zeros((N, D), dtype=torch.int64, device=DEV)
    W = case.cpu_weights()
    seqs = range(N) if seqs is None else seqs
    n_masked = []
    for t in range(n_passes):
        case.tokens = blk.clone()
        n_masked.append(int((conf == 0).sum()))
        print(f"refinement {wl.name} pass {t}: {n_masked[-1]} masked", flush=True)
        if t == 0:
            _, lg, st = case.step()
        else:
            ctx = case.ctx + (case.new if wl.ctx_source == "hidden" else 0)
            _, lg, st = case.call(ctx, np.zeros(N, np.int64), None)
        torch.cuda.synchronize()
        assert torch.all(st == 0)
        for i in seqs:
            toks, hid, kv = case.oracle_inputs(i)
            ref = od.drafter_forward(sh, W, toks, wl.n_anchor, hidden=hid, ctx_kv=kv)
            e = rel_l2(lg[i].cpu().numpy(), ref["logits"])
            assert e < TOL[sh.dtype], (t, i, e)
        blk, conf = _check_update(lg, blk, conf, wl.n_anchor, mask,
                                  refine.remask_count(D, n_passes, t + 1))
    assert n_masked == [N * refine.remask_count(D, n_passes, t) for t in range(n_passes)]
    assert torch.all(conf > 0)
    return blk


def test_refinement_loop_tiny_fp32():
    _loop(synth.workload("tiny-fp32"), 3)


def test_refinement_loop_bf16_wide_group():
    sh = synth.DrafterShape(hidden=512, n_q_heads=16, n_kv_heads=2, head_dim=64, ffn=1024,
                            n_layers=2, n_target_layers=2, vocab=2048, dtype="bf16")
    wl = synth.Workload(name="refine-bf16", shape=sh, batch=2, block_len=16, n_anchor=1,
                        n_drafts=1, temperature=0.0, ctx_lo=90, ctx_hi=130, ctx_source="hidden",
                        verify="greedy", verify_rows=16, planted_alpha=0.8, fixed_new=8)
    _loop(wl, 4)


def test_refinement_loop_cached_context_no_anchor():
    sh = synth.DrafterShape(hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=512,
                            n_layers=2, n_target_layers=0, vocab=1000, dtype="f32")
    wl = synth.Workload(name="refine-cache", shape=sh, batch=3, block_len=20, n_anchor=0,
                        n_drafts=1, temperature=0.0, ctx_lo=40, ctx_hi=70, ctx_source="cache",
                        verify="greedy", verify_rows=20, planted_alpha=0.8, fixed_new=0)
    _loop(wl, 3)
