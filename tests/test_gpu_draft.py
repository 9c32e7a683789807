"""GPU parity of draft_block against the fp64 oracle on the five workloads.

Floating outputs (cache K/V, per-layer residuals, logits) are compared by rel-L2: 1e-4 on the
fp32 path, 2e-2 on the bf16 path, for every sequence of the batch.  Drafted ids: top-1 agreement
with the oracle's argmax is reported; the ids draft_block returns must equal the oracle's
drafting (argmax, or the integer-exact sampler) applied to the fp32 logits draft_block returns,
bit for bit, and the verify or selection step that follows must equal the oracle's on the same
fp32 logits.  With DBD_PRECISION_DIR set, each end-to-end workload writes its figures to
precision_<workload>.json there."""
import json
import os

import numpy as np
import pytest
import torch

import block_diffusion_drafter_draft_amd as dbd
import synth
from oracle import accept, dnc, drafter as od
from drafter_case import Case, rel_l2

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = {"f32": 1e-4, "bf16": 2e-2}


def _compare(case, logits, seqs, report, residuals=True):
    """Cache K/V of every layer, the residual after every layer and the logits of the given
    sequences against the oracle; returns the per-sequence figures."""
    sh, wl = case.shape, case.wl
    W = case.oracle_weights()
    tol = TOL[sh.dtype]
    gres = case.residuals() if residuals else None
    rows = []
    for i in seqs:
        toks, hid, kv = case.oracle_inputs(i)
        ref = od.drafter_forward(sh, W, toks, wl.n_anchor, hidden=hid, ctx_kv=kv,
                                 keep=residuals)
        n_pos = int(case.ctx[i] + case.new[i])
        ek_l, ev_l, er_l = [], [], []
        for l in range(sh.n_layers):
            k, v = case.gpu_cache(i, l, n_pos)
            rk, rv = ref["ctx_kv"][l]
            ek, ev = rel_l2(k, od.f64(rk)), rel_l2(v, od.f64(rv))
            ek_l.append(ek)
            ev_l.append(ev)
            assert ek < tol and ev < tol, (i, l, ek, ev)
            if residuals:
                er = rel_l2(gres[l][i], ref["resid"][l])
                er_l.append(er)
                assert er < tol, ("residual", i, l, er)
        lg = logits[i].cpu().numpy()
        e = rel_l2(lg, ref["logits"])
        top = float(np.mean(lg.argmax(-1) == ref["logits"].argmax(-1)))
        rows.append({"seq": int(i), "ctx": int(case.ctx[i]), "new": int(case.new[i]),
                     "logits": e, "top1": top, "cache_k": ek_l, "cache_v": ev_l,
                     "resid": er_l})
        report.append((i, e, top))
        print(f"{wl.name} seq {i}: logits rel-L2 {e:.3e}, top-1 agreement {top:.3f}, cache max "
              f"{max(ek_l + ev_l):.2e}" + (f", residual max {max(er_l):.2e}" if er_l else ""),
              flush=True)
        assert e < tol, (i, e)
    return rows


def _check_drafts_property(case, drafts, logits):
    """The ids draft_block returns are its drafting stage applied to its own logits."""
    wl = case.wl
    if wl.temperature <= 0:
        assert np.array_equal(drafts[:, 0].cpu().numpy(), logits.cpu().numpy().argmax(-1))
    else:
        N, D, V = logits.shape
        ws = torch.empty(dbd.sample_workspace_bytes(N, D, V), dtype=torch.uint8, device=DEV)
        out = torch.empty_like(drafts)
        dbd.sample_from_logits(logits, wl.n_drafts, wl.temperature, 1234, out, ws)
        torch.cuda.synchronize()
        assert torch.equal(out, drafts)


def _exact_counts(case, drafts, logits):
    """Bit-exact agreement of the integer outputs on identical fp32 inputs: the drafts against
    the oracle's drafting of draft_block's own logits, then the workload's verify step (greedy
    verify, or streak selection and greedy accept) on planted verifier logits for those drafts,
    library against oracle.  Returns {output: [equal, total]}."""
    wl = case.wl
    N, K, D = drafts.shape
    V = case.shape.vocab
    lg = logits.cpu().numpy()
    ref = dnc.sample_drafts(lg, K, wl.temperature, 1234)
    got = drafts.cpu().numpy()
    out = {"drafts": [int(np.sum(got == ref)), int(got.size)]}
    assert np.array_equal(got, ref)
    if wl.verify == "streak":
        vl, _ = synth.make_planted_streak_logits(drafts, wl.verify_rows, V, wl.planted_alpha,
                                                 std=wl.logit_std, seed=5, device=DEV)
        ws = torch.empty(dbd.select_workspace_bytes(N, K, wl.verify_rows, V), dtype=torch.uint8,
                         device=DEV)
        sel = torch.empty(N, dtype=torch.int32, device=DEV)
        sc = torch.empty((N, K), dtype=torch.float64, device=DEV)
        na = torch.empty(N, dtype=torch.int32, device=DEV)
        bo = torch.empty(N, dtype=torch.int32, device=DEV)
        com = torch.empty((N, D + 1), dtype=torch.int32, device=DEV)
        dbd.select_streak(vl, drafts, sel, na, bo, com, ws, scores=sc)
        torch.cuda.synchronize()
        r = accept.select_streak(vl.cpu().numpy(), got)
        pairs = {"selected": (sel, r[0]), "scores": (sc, r[1]), "n_accepted": (na, r[2]),
                 "bonus": (bo, r[3]), "committed": (com, r[4])}
    else:
        d0 = drafts[:, 0].contiguous()
        vl, _ = synth.make_planted_verify_logits(d0, wl.verify_rows, V, wl.planted_alpha,
                                                 std=wl.logit_std, seed=5, device=DEV)
        ws = torch.empty(dbd.verify_workspace_bytes(N, wl.verify_rows, V), dtype=torch.uint8,
                         device=DEV)
        na = torch.empty(N, dtype=torch.int32, device=DEV)
        bo = torch.empty(N, dtype=torch.int32, device=DEV)
        com = torch.empty((N, D + 1), dtype=torch.int32, device=DEV)
        dbd.verify_greedy(vl, d0, na, bo, com, ws)
        torch.cuda.synchronize()
        r = accept.verify_greedy(vl.cpu().numpy(), got[:, 0])
        pairs = {"n_accepted": (na, r[0]), "bonus": (bo, r[1]), "committed": (com, r[2])}
    for name, (g, rr) in pairs.items():
        g = g.cpu().numpy()
        out[name] = [int(np.sum(g == rr)), int(g.size)]
        assert np.array_equal(g, rr), name
    return out


def _write_report(case, rows, exact, extra=None):
    d = os.environ.get("DBD_PRECISION_DIR")
    if not d:
        return
    wl, sh = case.wl, case.shape
    L = sh.n_layers

    def col(key, l):
        return max(r[key][l] for r in rows)
    rep = {
        "workload": wl.name, "dtype": sh.dtype, "act_pairs": wl.act_pairs, "batch": wl.batch,
        "sequences_compared": len(rows), "rel_l2_bar": TOL[sh.dtype],
        "oracle": "oracle.drafter.drafter_forward (fp64, stateless: context K/V recomputed "
                  "from every context position)",
        "logits_rel_l2": {"max": max(r["logits"] for r in rows),
                          "mean": float(np.mean([r["logits"] for r in rows]))},
        "top1_agreement": {"min": min(r["top1"] for r in rows),
                           "mean": float(np.mean([r["top1"] for r in rows]))},
        "cache_k_rel_l2_max_per_layer": [col("cache_k", l) for l in range(L)],
        "cache_v_rel_l2_max_per_layer": [col("cache_v", l) for l in range(L)],
        "residual_rel_l2_max_per_layer": ([col("resid", l) for l in range(L)]
                                          if rows[0]["resid"] else None),
        "bit_exact_equal_of_total": exact,
        "per_sequence": [{k: r[k] for k in ("seq", "ctx", "new", "logits", "top1")}
                         for r in rows],
    }
    if extra:
        rep.update(extra)
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, f"precision_{wl.name}.json"), "w") as f:
        json.dump(rep, f, indent=1)


def _ctx_feature_errors(case):
    """rel-L2 of the mixing stage (bf16 or fp32 output of the library's mix kernel) against the
    oracle's fp64 context features, per draft layer, over the step's ingested rows."""
    sh = case.shape
    if sh.n_target_layers == 0 or getattr(sh, "ctx_fusion", "mix") != "mix":
        return None
    h = case._hidden_rows(case.ctx, case.ctx + case.new)
    if h.numel() == 0:
        return None
    out = torch.empty((sh.n_layers, h.shape[0], sh.hidden), dtype=h.dtype, device=DEV)
    dbd.mix_rmsnorm(case.desc, case.W["mix_logits"], case.W["mix_norm_w"], h, out)
    torch.cuda.synchronize()
    W = case.oracle_weights()
    hc = h.cpu()
    return [rel_l2(out[l].float().cpu().numpy(), od.context_features(sh, W, l, hc))
            for l in range(sh.n_layers)]


def _run(name, seqs=None, **kw):
    wl = synth.workload(name)
    print(f"draft_block workload={name}", flush=True)
    case = Case(wl, dev=DEV, **kw)
    case.fill_cache()
    drafts, logits, status = case.step()
    torch.cuda.synchronize()
    assert torch.all(status == 0)
    assert int(drafts.min()) >= 0 and int(drafts.max()) < wl.shape.vocab
    _check_drafts_property(case, drafts, logits)
    exact = _exact_counts(case, drafts, logits)
    report = []
    rows = _compare(case, logits, seqs if seqs is not None else range(wl.batch), report)
    cf = _ctx_feature_errors(case)
    _write_report(case, rows, exact, {"ctx_features_rel_l2_per_layer": cf} if cf else None)
    return case, drafts, logits


def test_tiny_fp32_matches_oracle():
    case, drafts, logits = _run("tiny-fp32")
    # fp32 end to end: the argmax drafts agree with the oracle's
    toks, hid, kv = case.oracle_inputs(0)
    ref = od.drafter_forward(case.shape, case.cpu_weights(), toks, 1, hidden=hid)
    assert np.array_equal(drafts[0, 0].cpu().numpy(), ref["logits"].argmax(-1))


def test_tiny_fp32_cold_ingest_equals_incremental():
    wl = synth.workload("tiny-fp32")
    case = Case(wl, dev=DEV)
    case.fill_cache()
    d1, l1, _ = case.step()
    case2 = Case(wl, dev=DEV, ctx=np.zeros(1, np.int64), new=case.ctx + case.new)
    d2, l2, _ = case2.step()
    torch.cuda.synchronize()
    assert torch.equal(l1, l2) and torch.equal(d1, d2)
    n = int(case.ctx[0] + case.new[0])
    assert torch.equal(case.kv_k[:, :, :, :n], case2.kv_k[:, :, :, :n])


@pytest.mark.parametrize("name", ["tiny-fp32", "qwen3-4b"])
def test_step_is_deterministic_and_idempotent(name):
    wl = synth.workload(name)
    case = Case(wl, dev=DEV)
    case.fill_cache()
    d1, l1, _ = case.step()
    d2, l2, _ = case.step()                 # same ctx_len: re-ingest overwrites identically
    torch.cuda.synchronize()
    assert torch.equal(l1, l2) and torch.equal(d1, d2)


def test_tiny_sampling_and_multiple_drafts():
    wl = synth.workload("tiny-fp32").with_(n_drafts=4, temperature=1.0)
    case = Case(wl, dev=DEV)
    case.fill_cache()
    drafts, logits, status = case.step()
    torch.cuda.synchronize()
    assert drafts.shape == (1, 4, 7)
    _check_drafts_property(case, drafts, logits)
    _compare(case, logits, [0], [])


def test_bad_lengths_are_flagged_and_skipped():
    wl = synth.workload("tiny-fp32").with_(batch=3, ctx_lo=10, ctx_hi=20)
    case = Case(wl, dev=DEV)
    case.fill_cache()
    ctx = case.ctx.copy()
    ctx[1] = case.cap                        # block would not fit the cache
    off = torch.tensor([0, 0, 0, 0], dtype=torch.int32, device=DEV)
    ws = case.workspace(0, 1, 0.0)
    out = torch.full((3, 1, 7), -7, dtype=torch.int32, device=DEV)
    st = torch.full((3,), -7, dtype=torch.int32, device=DEV)
    before = case.kv_k[:, 1].clone()
    dbd.draft_block(case.desc, case.wstruct, case.tokens, None, off,
                    torch.tensor(ctx.astype(np.int32), device=DEV), case.kv_k, case.kv_v, out,
                    ws, 0, seq_status=st)
    torch.cuda.synchronize()
    assert st.tolist() == [0, dbd.SEQ_BAD_LENGTH, 0]
    assert torch.all(out[1] == -1) and torch.all(out[0] >= 0) and torch.all(out[2] >= 0)
    assert torch.equal(case.kv_k[:, 1], before)


def test_qwen3_4b_matches_oracle():
    _run("qwen3-4b")


def test_activation_pairs_are_more_accurate():
    """The same Qwen3-4B-shaped step with bf16 activation pairs is closer to the oracle than with
    plain bf16 activations, and still within tolerance."""
    errs = {}
    for pairs in (0, 1):
        wl = synth.workload("qwen3-4b").with_(act_pairs=pairs)
        case = Case(wl, dev=DEV)
        case.fill_cache()
        drafts, logits, status = case.step()
        torch.cuda.synchronize()
        _check_drafts_property(case, drafts, logits)
        report = []
        _compare(case, logits, [0], report)
        errs[pairs] = report[0][1]
    print(f"qwen3-4b logits rel-L2: plain bf16 {errs[0]:.3e}, pairs {errs[1]:.3e}", flush=True)
    assert errs[1] < 0.75 * errs[0]          # the K/V cache and P stay bf16 in both modes


@pytest.mark.timeout(900)
def test_qwen3_8b_every_sequence_matches_oracle():
    _run("qwen3-8b")


@pytest.mark.timeout(900)
def test_gpt_oss_20b_every_sequence_matches_oracle():
    _run("gpt-oss-20b")


@pytest.mark.timeout(900)
def test_specdiff2_7b_every_sequence_matches_oracle():
    _run("specdiff2-7b")


@pytest.mark.parametrize("name", ["tiny-dflash-fp32", "tiny-ablate-fp32"])
def test_context_path_variants_fp32_match_oracle(name):
    """Fully connected fusion with the shared K/V projection, and mixing without softmax with the
    shared projection: cache K/V and logits within 1e-4 of the oracle, argmax drafts equal."""
    case, drafts, logits = _run(name)
    toks, hid, kv = case.oracle_inputs(0)
    ref = od.drafter_forward(case.shape, case.cpu_weights(), toks, 1, hidden=hid)
    assert np.array_equal(drafts[0, 0].cpu().numpy(), ref["logits"].argmax(-1))


def test_tiny_dflash_cold_ingest_equals_incremental():
    wl = synth.workload("tiny-dflash-fp32")
    case = Case(wl, dev=DEV)
    case.fill_cache()
    d1, l1, _ = case.step()
    case2 = Case(wl, dev=DEV, ctx=np.zeros(1, np.int64), new=case.ctx + case.new)
    d2, l2, _ = case2.step()
    torch.cuda.synchronize()
    assert torch.equal(l1, l2) and torch.equal(d1, d2)


@pytest.mark.timeout(900)
def test_qwen3_8b_dflash_every_sequence_matches_oracle():
    """The bench workload with the fully connected context fusion, bf16, every sequence."""
    _run("qwen3-8b-dflash")


def test_query_groups_beyond_one_workgroup_match_oracle():
    """8 query heads per kv head and a 40-position block: 320 query rows per kv head, more than
    one attention workgroup holds, so two row blocks read the same keys (bf16 path)."""
    sh = synth.DrafterShape(hidden=512, n_q_heads=16, n_kv_heads=2, head_dim=64, ffn=1024,
                            n_layers=2, n_target_layers=2, vocab=2048, dtype="bf16")
    wl = synth.Workload(name="wide-group", shape=sh, batch=2, block_len=40, n_anchor=1,
                        n_drafts=1, temperature=0.0, ctx_lo=90, ctx_hi=130, ctx_source="hidden",
                        verify="greedy", verify_rows=40, planted_alpha=0.8, fixed_new=8)
    print("draft_block workload=wide-group", flush=True)
    case = Case(wl, dev=DEV)
    case.fill_cache()
    drafts, logits, status = case.step()
    torch.cuda.synchronize()
    assert torch.all(status == 0)
    _check_drafts_property(case, drafts, logits)
    _compare(case, logits, range(wl.batch), [])


@pytest.mark.parametrize("workgroups,depth", [(1, 1), (3, 2), (7, 1), (64, 2), (2048, 2),
                                               (0, 1)])
def test_attention_workgroup_and_depth_overrides_match_oracle(workgroups, depth):
    """The balanced attention with the workgroup count and load-ahead depth set by the tuning
    override: one workgroup walking every segment (whole segments only, no partials), a few
    workgroups whose ranges end inside segments (partials merged by the combine kernel), and
    more workgroups than chunks (empty ranges, segments spread over many pieces).  320 query rows
    per kv head (five row blocks), head size 64, contexts of 90-130 positions."""
    sh = synth.DrafterShape(hidden=512, n_q_heads=16, n_kv_heads=2, head_dim=64, ffn=1024,
                            n_layers=2, n_target_layers=2, vocab=2048, dtype="bf16")
    wl = synth.Workload(name="attn-override", shape=sh, batch=3, block_len=40, n_anchor=1,
                        n_drafts=1, temperature=0.0, ctx_lo=90, ctx_hi=130, ctx_source="hidden",
                        verify="greedy", verify_rows=40, planted_alpha=0.8, fixed_new=8)
    print(f"draft_block workload=attn-override workgroups={workgroups} depth={depth}", flush=True)
    dbd.attn_override(workgroups, depth)
    try:
        case = Case(wl, dev=DEV)
        case.fill_cache()
        drafts, logits, status = case.step()
        torch.cuda.synchronize()
        assert torch.all(status == 0)
        _check_drafts_property(case, drafts, logits)
        _compare(case, logits, range(wl.batch), [], residuals=False)
    finally:
        dbd.attn_override(0, 0)


PAIR_ROW_OVERRIDES = [
    {},
    {"gemm_qkv": (16, 3), "gemm_o": (16, 2), "gemm_gateup": (15, 2), "gemm_down": (16, 4),
     "gemm_lmhead": (14, 1)},
    {"gemm_qkv": (16, 1), "gemm_o": (14, 3), "gemm_gateup": (14, 1), "gemm_down": (15, 2),
     "gemm_lmhead": (16, 2)},
]


@pytest.mark.parametrize("batch", [5, 8])
@pytest.mark.parametrize("ov", range(len(PAIR_ROW_OVERRIDES)))
def test_pair_rows_tiles_match_oracle(batch, ov):
    """bf16 activation pairs on 80 and 128 block rows: the register-staged 256-row tiles take
    the pair as rows (high part, low part) and add them per output row, unsplit and with split K
    (the reduction folds the two halves), under every projection's epilogue (rotation and cache
    write, residual, SwiGLU, LM-head argmax)."""
    sh = synth.DrafterShape(hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=64, ffn=1536,
                            n_layers=2, n_target_layers=2, vocab=3000, dtype="bf16")
    wl = synth.Workload(name="pair-rows", shape=sh, batch=batch, block_len=16, n_anchor=1,
                        n_drafts=1, temperature=0.0, ctx_lo=60, ctx_hi=140, ctx_source="hidden",
                        verify="greedy", verify_rows=16, planted_alpha=0.8, fixed_new=4,
                        act_pairs=1)
    print(f"draft_block workload=pair-rows batch={batch} overrides={PAIR_ROW_OVERRIDES[ov]}",
          flush=True)
    for st, (cfg, sp) in PAIR_ROW_OVERRIDES[ov].items():
        dbd.gemm_override(st, cfg, sp)
    try:
        case = Case(wl, dev=DEV)
        case.fill_cache()
        drafts, logits, status = case.step()
        torch.cuda.synchronize()
        assert torch.all(status == 0)
        _check_drafts_property(case, drafts, logits)
        _compare(case, logits, range(wl.batch), [], residuals=False)
    finally:
        for st in PAIR_ROW_OVERRIDES[ov]:
            dbd.gemm_override(st, -1, 0)


@pytest.mark.parametrize("vocab", [3000, 200])
@pytest.mark.parametrize("batch", [5, 20])
@pytest.mark.parametrize("cfg", [None, 14, 15, 16])
def test_lm_head_argmax_without_logits_matches(batch, cfg, vocab):
    """Greedy drafting with no logits output: the register-staged LM-head tiles (256, 192 and
    128 columns, unsplit) then take each row's argmax straight from their accumulators instead
    of from the tile staged in LDS.  75 and 300 block rows (one and two row tiles, ragged) over
    a 3,000-token vocabulary (a ragged last column tile for every width) and a 200-token one
    (a single column tile, in which the 256-column tile's last wave along N sees no column of
    the vocabulary): the drafts equal those of the same step with logits, which equal the
    argmax of those logits, which match the oracle."""
    sh = synth.DrafterShape(hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=64, ffn=1024,
                            n_layers=2, n_target_layers=2, vocab=vocab, dtype="bf16")
    wl = synth.Workload(name="lm-head-argmax", shape=sh, batch=batch, block_len=16, n_anchor=1,
                        n_drafts=1, temperature=0.0, ctx_lo=60, ctx_hi=140, ctx_source="hidden",
                        verify="greedy", verify_rows=16, planted_alpha=0.8, fixed_new=4)
    print(f"draft_block workload=lm-head-argmax batch={batch} lmhead_cfg={cfg} vocab={vocab}",
          flush=True)
    if cfg is not None:
        dbd.gemm_override("gemm_lmhead", cfg, 1)
    try:
        case = Case(wl, dev=DEV)
        case.fill_cache()
        drafts, logits, status = case.step()
        torch.cuda.synchronize()
        assert torch.all(status == 0)
        _check_drafts_property(case, drafts, logits)
        _compare(case, logits, range(wl.batch), [], residuals=False)
        drafts2, none, status2 = case.step(logits=False)
        torch.cuda.synchronize()
        assert none is None and torch.all(status2 == 0)
        assert torch.equal(drafts, drafts2)
    finally:
        if cfg is not None:
            dbd.gemm_override("gemm_lmhead", -1, 0)


@pytest.mark.parametrize("cfg", [14, 15, 16])
def test_lm_head_argmax_ties_go_to_the_lowest_index(cfg):
    """Every LM-head weight row repeats row v mod 37, so each logit row takes 37 distinct values
    and its maximum sits at about 81 columns (in every lane group, wave and column tile of the
    tile), all bit-identical.  The draft is the lowest of them, so it is below 37, with and
    without logits (the register argmax then folds the ties in another order)."""
    sh = synth.DrafterShape(hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=64, ffn=1024,
                            n_layers=2, n_target_layers=2, vocab=3000, dtype="bf16")
    wl = synth.Workload(name="lm-head-ties", shape=sh, batch=20, block_len=16, n_anchor=1,
                        n_drafts=1, temperature=0.0, ctx_lo=60, ctx_hi=140, ctx_source="hidden",
                        verify="greedy", verify_rows=16, planted_alpha=0.8, fixed_new=4)
    print(f"draft_block workload=lm-head-ties lmhead_cfg={cfg}", flush=True)
    dbd.gemm_override("gemm_lmhead", cfg, 1)
    try:
        case = Case(wl, dev=DEV)
        lm = case.W["lm_head"]
        lm.copy_(lm[torch.arange(sh.vocab, device=DEV) % 37].clone())
        case.fill_cache()
        drafts, logits, status = case.step()
        torch.cuda.synchronize()
        assert torch.all(status == 0)
        _check_drafts_property(case, drafts, logits)
        lg = logits.cpu().numpy()
        assert np.array_equal(lg[..., :37], lg[..., 37:74])
        drafts2, _, status2 = case.step(logits=False)
        torch.cuda.synchronize()
        assert torch.all(status2 == 0)
        assert torch.equal(drafts, drafts2)
        d = drafts2[:, 0].cpu().numpy()
        d = d[d >= 0]                                   # -1 marks rows past a sequence's end
        assert d.size > 0 and d.max() < 37, d.max()
    finally:
        dbd.gemm_override("gemm_lmhead", -1, 0)


@pytest.mark.parametrize("name", ["qwen3-4b-tiny-batch", "specdiff-tiny-batch"])
@pytest.mark.parametrize("workgroups", [1, 5])
def test_sequence_placement_in_the_batch_is_invisible(name, workgroups):
    """Every sequence's result depends on that sequence only, up to where the balanced attention
    cuts its key chunks: the same three sequences in another order in the batch (same batch size
    and capacity, so the same GEMM tiles and splits).  With one attention workgroup every
    segment is computed whole, so logits, cache contents and argmax drafts are bit-identical.
    With five workgroups the cuts depend on the lengths of the sequences before it in the batch
    (as they do at the library's workgroup count once a batch has more chunks than workgroups),
    so the partials merge in another grouping and the attention outputs differ in their last
    bits.  Every single-bf16 rounding downstream (the block's keys and values in the cache, and
    the activations without pairs) turns that into flipped roundings, each moving an element by
    2^-8 of itself, so the two orders agree only to the bf16 path's own accuracy: one order
    matches the oracle within its tolerance and the two match each other within the same
    tolerance (measured 5e-3 without activation pairs and 1.1e-3 with them, against 2e-3 to 1e-2
    from the oracle)."""
    if name == "qwen3-4b-tiny-batch":
        sh = synth.DrafterShape(hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=64, ffn=1024,
                                n_layers=2, n_target_layers=3, vocab=2048, dtype="bf16")
        wl = synth.Workload(name=name, shape=sh, batch=3, block_len=16, n_anchor=1, n_drafts=1,
                            temperature=0.0, ctx_lo=40, ctx_hi=300, ctx_source="hidden",
                            verify="greedy", verify_rows=16, planted_alpha=0.8)
    else:
        sh = synth.DrafterShape(hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=1024,
                                n_layers=2, n_target_layers=0, vocab=2048, dtype="bf16")
        wl = synth.Workload(name=name, shape=sh, batch=3, block_len=32, n_anchor=0, n_drafts=4,
                            temperature=1.5, ctx_lo=50, ctx_hi=400, ctx_source="cache",
                            verify="streak", verify_rows=32, planted_alpha=0.8, fixed_new=0,
                            act_pairs=1)
    print(f"draft_block workload={name} placement workgroups={workgroups}", flush=True)
    dbd.attn_override(workgroups, 0)
    try:
        _placement(wl, workgroups == 1)
    finally:
        dbd.attn_override(0, 0)


def _placement(wl, exact):
    a = Case(wl, dev=DEV)
    perm = [2, 0, 1]
    b = Case(wl, dev=DEV)
    assert b.cap == a.cap
    b.tokens = a.tokens[perm].contiguous()
    b.ctx, b.new = a.ctx[perm], a.new[perm]
    if wl.ctx_source == "hidden":
        b.hidden = [a.hidden[i] for i in perm]
    else:
        b.kv_k.copy_(a.kv_k[:, perm])
        b.kv_v.copy_(a.kv_v[:, perm])
    a.fill_cache()
    b.fill_cache()
    da, la, sa = a.step()
    db_, lb, sb = b.step()
    torch.cuda.synchronize()
    assert torch.all(sa == 0) and torch.all(sb == 0)
    if not exact:
        # the oracle inputs of `b` are those it was generated with, not the permuted copies of
        # `a`'s, so only `a` is compared with the oracle
        _check_drafts_property(a, da, la)
        _check_drafts_property(b, db_, lb)
        _compare(a, la, range(wl.batch), [], residuals=False)
    bound = TOL[wl.shape.dtype]
    for j, i in enumerate(perm):
        n = int(a.ctx[i] + a.new[i])
        if exact:
            assert torch.equal(la[i], lb[j]), (i, j)
            if wl.temperature <= 0:
                assert torch.equal(da[i], db_[j]), (i, j)
            assert torch.equal(a.kv_k[:, i, :, :n], b.kv_k[:, j, :, :n])
            continue
        x, y = la[i].double(), lb[j].double()
        rel = float((x - y).norm() / x.norm())
        print(f"placement seq {i}: logits rel-L2 between the two orders {rel:.3e}", flush=True)
        assert rel < bound, (i, j, rel)


@pytest.mark.parametrize("pairs", [0, 1])
def test_small_block_fused_residual_norm_matches_oracle(pairs):
    """32 block rows with K large enough that the O and down projections take the skinny tiles
    with a split K (O split 2, down split 4): their split reduction also writes the next RMSNorm
    (the MLP norm, the next layer's attention norm, after the last layer the final norm of the
    mask rows, compacted) and no separate norm runs.  With bf16 activation pairs the fused
    reduction writes the low parts too."""
    sh = synth.DrafterShape(hidden=1024, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=2048,
                            n_layers=3, n_target_layers=2, vocab=2048, dtype="bf16")
    wl = synth.Workload(name="fused-norm", shape=sh, batch=2, block_len=16, n_anchor=1,
                        n_drafts=1, temperature=0.0, ctx_lo=60, ctx_hi=140, ctx_source="hidden",
                        verify="greedy", verify_rows=16, planted_alpha=0.8, fixed_new=8,
                        act_pairs=pairs)
    print(f"draft_block workload=fused-norm pairs={pairs}", flush=True)
    case = Case(wl, dev=DEV)
    case.fill_cache()
    drafts, logits, status = case.step()
    torch.cuda.synchronize()
    assert torch.all(status == 0)
    _check_drafts_property(case, drafts, logits)
    _compare(case, logits, range(wl.batch), [])
    # the row-norm stage keeps only the embedding (which writes the first layer's attention
    # norm); the last down projection writes the final norm of the mask rows
    dbd.timing_reset()
    dbd.timing_enable(True)
    try:
        _, logits2, _ = case.step()
        torch.cuda.synchronize()
        launches = dbd.timing_read()["rownorm"][1]
    finally:
        dbd.timing_enable(False)
        dbd.timing_reset()
    assert launches == 1, launches
    assert torch.equal(logits, logits2)


FUSED_NORM_OVERRIDES = [
    ({"gemm_o": (16, 4), "gemm_down": (16, 3)}, 0),
    ({"gemm_o": (15, 2), "gemm_down": (14, 5)}, 0),
    ({"gemm_o": (8, 2), "gemm_down": (9, 3)}, 0),
    ({"gemm_o": (10, 2), "gemm_down": (10, 4)}, 1),
]


@pytest.mark.parametrize("batch", [13, 20])
@pytest.mark.parametrize("ov", range(len(FUSED_NORM_OVERRIDES)))
def test_register_staged_fused_residual_norm_matches_oracle(batch, ov):
    """208 and 320 block rows (a ragged last row tile) with the O and down projections split
    along K on the register-staged 256-row tiles (128-, 192- and 256-column tiles; 1,024 columns
    leave a ragged 192-column tile) and on the four-wave deep-ring tiles (256 x 128, 128 x 256,
    and 128 x 128 with the bf16 activation pair as a second A part): their units store row-major
    partials and the fused reduction writes the residual and the next RMSNorm (the final norm of
    the mask rows after the last layer), so the row-norm stage keeps only the embedding, which
    writes the first layer's attention norm."""
    ovs, pairs = FUSED_NORM_OVERRIDES[ov]
    sh = synth.DrafterShape(hidden=1024, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=2048,
                            n_layers=3, n_target_layers=2, vocab=2048, dtype="bf16")
    wl = synth.Workload(name="fused-norm-w8r", shape=sh, batch=batch, block_len=16, n_anchor=1,
                        n_drafts=1, temperature=0.0, ctx_lo=60, ctx_hi=140, ctx_source="hidden",
                        verify="greedy", verify_rows=16, planted_alpha=0.8, fixed_new=8,
                        act_pairs=pairs)
    print(f"draft_block workload=fused-norm-w8r batch={batch} overrides={ovs} pairs={pairs}",
          flush=True)
    for st, (cfg, sp) in ovs.items():
        dbd.gemm_override(st, cfg, sp)
    try:
        case = Case(wl, dev=DEV)
        case.fill_cache()
        drafts, logits, status = case.step()
        torch.cuda.synchronize()
        assert torch.all(status == 0)
        _check_drafts_property(case, drafts, logits)
        _compare(case, logits, range(wl.batch), [])
        dbd.timing_reset()
        dbd.timing_enable(True)
        try:
            _, logits2, _ = case.step()
            torch.cuda.synchronize()
            launches = dbd.timing_read()["rownorm"][1]
        finally:
            dbd.timing_enable(False)
            dbd.timing_reset()
        assert launches == 1, launches
        assert torch.equal(logits, logits2)
    finally:
        for st in ovs:
            dbd.gemm_override(st, -1, 0)


def test_long_context_single_sequence_many_splits():
    """One sequence over a 716-position cache: 12 key chunks per kv head, fewer chunks than
    attention workgroups, so every chunk is a piece of its own and the combine kernel merges
    twelve partials per row (more than one round of its eight loads in flight)."""
    sh = synth.DrafterShape(hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=1024,
                            n_layers=2, n_target_layers=0, vocab=2048, dtype="bf16")
    wl = synth.Workload(name="long-ctx", shape=sh, batch=1, block_len=16, n_anchor=1,
                        n_drafts=1, temperature=0.0, ctx_lo=700, ctx_hi=700, ctx_source="cache",
                        verify="greedy", verify_rows=16, planted_alpha=0.8, fixed_new=0)
    print("draft_block workload=long-ctx", flush=True)
    case = Case(wl, dev=DEV)
    drafts, logits, status = case.step()
    torch.cuda.synchronize()
    assert torch.all(status == 0)
    _check_drafts_property(case, drafts, logits)
    _compare(case, logits, range(wl.batch), [])


def test_sixty_four_mask_block_without_anchor():
    """block_len 64 (the interface's maximum), all masks, context from a given cache, 7 query
    heads per kv head: 448 query rows per kv head over two attention row blocks."""
    sh = synth.DrafterShape(hidden=896, n_q_heads=7, n_kv_heads=1, head_dim=128, ffn=1536,
                            n_layers=2, n_target_layers=0, vocab=3000, dtype="bf16")
    wl = synth.Workload(name="block64", shape=sh, batch=2, block_len=64, n_anchor=0, n_drafts=4,
                        temperature=1.5, ctx_lo=70, ctx_hi=70, ctx_source="cache",
                        verify="streak", verify_rows=64, planted_alpha=0.8, fixed_new=0)
    print("draft_block workload=block64", flush=True)
    case = Case(wl, dev=DEV)
    drafts, logits, status = case.step()
    torch.cuda.synchronize()
    assert torch.all(status == 0)
    _check_drafts_property(case, drafts, logits)
    _compare(case, logits, range(wl.batch), [])


def test_step_replays_from_a_hip_graph():
    """A sampling draft_block (ingest + block forward + 4 joint drafts) and verify_greedy, captured
    once in a HIP graph: every replay, with eager library calls and torch work between replays,
    gives the eager call's drafts, logits, status and acceptance bit for bit."""
    sh = synth.DrafterShape(hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=64, ffn=1024,
                            n_layers=2, n_target_layers=2, vocab=2048, dtype="bf16")
    wl = synth.Workload(name="graph", shape=sh, batch=3, block_len=16, n_anchor=1, n_drafts=4,
                        temperature=1.2, ctx_lo=70, ctx_hi=130, ctx_source="hidden",
                        verify="greedy", verify_rows=16, planted_alpha=0.8, fixed_new=5)
    print("draft_block + verify_greedy under graph capture", flush=True)
    case = Case(wl, dev=DEV)
    case.fill_cache()
    N, D, V, K = wl.batch, case.D, sh.vocab, wl.n_drafts
    hid = case._hidden_rows(case.ctx, case.ctx + case.new)
    off, tot = case._offsets(case.new)
    ctx = torch.tensor(case.ctx.astype(np.int32), device=DEV)
    ws = case.workspace(tot, K, wl.temperature)
    drafts = torch.empty((N, K, D), dtype=torch.int32, device=DEV)
    logits = torch.empty((N, D, V), dtype=torch.float32, device=DEV)
    status = torch.empty((N,), dtype=torch.int32, device=DEV)
    tl, _ = synth.make_planted_verify_logits(synth.make_drafts(N, 1, D, V, seed=3, device=DEV)[:, 0]
                                             .contiguous(), wl.verify_rows, V, 0.8, seed=3,
                                             device=DEV)
    vws = torch.empty(dbd.verify_workspace_bytes(N, wl.verify_rows, V), dtype=torch.uint8,
                      device=DEV)
    n_acc = torch.empty((N,), dtype=torch.int32, device=DEV)
    bonus = torch.empty((N,), dtype=torch.int32, device=DEV)
    com = torch.empty((N, D + 1), dtype=torch.int32, device=DEV)
    outs = (drafts, logits, status, n_acc, bonus, com)

    def run():
        dbd.draft_block(case.desc, case.wstruct, case.tokens, hid, off, ctx, case.kv_k,
                        case.kv_v, drafts, ws, tot, n_drafts=K, temperature=wl.temperature,
                        seed=99, n_anchor=wl.n_anchor, logits_out=logits, seq_status=status)
        dbd.verify_greedy(tl, drafts[:, 0], n_acc, bonus, com, vws)

    run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for rep in range(4):
        for t in outs:
            t.fill_(-3)
        graph.replay()
        torch.cuda.synchronize()
        for t, r in zip(outs, ref):
            assert torch.equal(t, r), f"replay {rep} differs"
        run()                                     # eager work between replays
        torch.cuda.synchronize()
    assert torch.all(status == 0)
