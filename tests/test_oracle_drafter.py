"""Pins of the fp64 drafter oracle (oracle/drafter.py): closed forms, invariants, special cases
and brute force.  The composed forward pass has no worked example on the pages, so beyond these
pins of its parts it is "parity unpinned".  CPU only."""
import json
import math
import os

import numpy as np
import pytest

from oracle import drafter as od
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TINY = synth.workload("tiny-fp32").shape


@pytest.fixture(scope="module")
def tiny_w():
    return {k: v.numpy() for k, v in synth.make_weights(TINY, seed=0).items()}


def _hidden(n, seq=0, start=0):
    return synth.make_hidden(TINY, n, seed=0, seq=seq, start=start).numpy()


# ---- mixing + RMSNorm -------------------------------------------------------------------------

def test_mix_weights_sum_to_one(tiny_w):
    w = od.mix_weights(tiny_w["mix_logits"])
    assert w.shape == (TINY.n_layers, TINY.n_target_layers)
    assert np.all(np.abs(w.sum(1) - 1.0) < 1e-15) and np.all(w > 0)


def test_one_hot_mix_selects_one_target_layer(tiny_w):
    h = _hidden(10)
    for i in range(TINY.n_target_layers):
        W = dict(tiny_w)
        lg = np.zeros_like(W["mix_logits"])
        lg[:, i] = 1e4
        W["mix_logits"] = lg
        for l in range(TINY.n_layers):
            c = od.context_features(TINY, W, l, h)
            # w = (1, 0, 0) exactly in fp64, so the mix is h_i bit for bit
            ref = od.rmsnorm(h[:, i, :].astype(np.float64), W["mix_norm_w"][l], TINY.rms_eps)
            assert np.array_equal(c, ref)


def test_equal_mix_logits_give_the_mean(tiny_w):
    h = _hidden(5)
    W = dict(tiny_w)
    W["mix_logits"] = np.full_like(W["mix_logits"], 0.3)
    c = od.context_features(TINY, W, 0, h)
    mean = h.astype(np.float64).mean(axis=1)
    ref = od.rmsnorm(mean, W["mix_norm_w"][0], TINY.rms_eps)
    assert np.max(np.abs(c - ref)) < 1e-12


def test_mixing_is_permutation_invariant(tiny_w):
    h = _hidden(6)
    perm = np.array([2, 0, 1])
    W2 = dict(tiny_w)
    W2["mix_logits"] = tiny_w["mix_logits"][:, perm]
    a = od.context_features(TINY, tiny_w, 1, h)
    b = od.context_features(TINY, W2, 1, h[:, perm, :])
    assert np.max(np.abs(a - b)) < 1e-12


def test_rmsnorm_closed_form():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 33)) * rng.uniform(0.01, 10, size=(7, 1))
    eps = 1e-6
    y = od.rmsnorm(x, np.ones(33), eps)
    ms = np.mean(x * x, axis=1)
    assert np.allclose(np.mean(y * y, axis=1), ms / (ms + eps), rtol=1e-13, atol=0)
    # direction is kept, the gain multiplies element-wise
    g = rng.uniform(0.5, 1.5, 33)
    assert np.allclose(od.rmsnorm(x, g, eps), y * g, rtol=1e-14)
    assert np.all(np.sign(y) == np.sign(x))


# ---- RoPE ---------------------------------------------------------------------------------------

def test_rope_position_zero_is_identity():
    x = np.random.default_rng(1).standard_normal((1, 3, 64))
    assert np.array_equal(od.rope(x, [0], 1e6), x)


def test_rope_two_dims_is_complex_rotation():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 1, 2))
    pos = np.array([0, 1, 7, 100, 4000])
    y = od.rope(x, pos, 1e6)
    z = (x[:, 0, 0] + 1j * x[:, 0, 1]) * np.exp(1j * pos)
    assert np.allclose(y[:, 0, 0], z.real, atol=1e-12) and np.allclose(y[:, 0, 1], z.imag,
                                                                         atol=1e-12)


def test_rope_relative_position_property():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 1, 128))
    k = rng.standard_normal((1, 1, 128))
    for p1, p2, s in [(5, 3, 100), (0, 17, 2000), (3000, 10, 77)]:
        a = np.dot(od.rope(q, [p1], 1e6)[0, 0], od.rope(k, [p2], 1e6)[0, 0])
        b = np.dot(od.rope(q, [p1 + s], 1e6)[0, 0], od.rope(k, [p2 + s], 1e6)[0, 0])
        assert abs(a - b) < 1e-9
        assert abs(np.linalg.norm(od.rope(q, [p1], 1e6)) - np.linalg.norm(q)) < 1e-12


def _rope_by_hand(x, p, inv_freq):
    """Rotate-half written out element by element: dimension i (i < hd/2) is paired with
    i + hd/2, and the pair turns by the angle p * inv_freq[i]."""
    hd = len(x)
    half = hd // 2
    y = [0.0] * hd
    for i in range(half):
        a = p * inv_freq[i]
        y[i] = x[i] * math.cos(a) - x[i + half] * math.sin(a)
        y[i + half] = x[i + half] * math.cos(a) + x[i] * math.sin(a)
    return np.array(y)


def test_rope_frequency_schedule_and_pairing_by_hand():
    """Theta = 1e6: with head_dim 4 the two pair frequencies are 1 and 1e6^(-1/2) = 1e-3; with
    head_dim 8 they are 1, 10^-1.5, 10^-3 and 10^-4.5 (theta^(-2i/hd) for i = 0..hd/2-1).  These
    values are written out here as literals, so a schedule without the factor 2 (theta^(-i/hd))
    or pairs (2i, 2i+1) instead of (i, i+hd/2) fail."""
    rng = np.random.default_rng(11)
    schedules = {4: [1.0, 1e-3], 8: [1.0, 10 ** -1.5, 1e-3, 10 ** -4.5]}
    for hd, inv_freq in schedules.items():
        x = rng.standard_normal((3, 2, hd))
        pos = [1, 7, 3000]
        y = od.rope(x, pos, 1e6)
        for t, p in enumerate(pos):
            for h in range(2):
                ref = _rope_by_hand(list(x[t, h]), p, inv_freq)
                assert np.max(np.abs(y[t, h] - ref)) < 1e-12, (hd, p)


def test_rope_first_pair_at_position_one_turns_by_one_radian():
    """Frequency 1 for the first pair means position 1 turns (x_0, x_{hd/2}) by exactly one
    radian; the second half of a unit vector e_{hd/2} goes to (-sin 1, cos 1)."""
    hd = 8
    e = np.zeros((1, 1, hd))
    e[0, 0, hd // 2] = 1.0
    y = od.rope(e, [1], 1e6)[0, 0]
    assert abs(y[0] + math.sin(1.0)) < 1e-15 and abs(y[hd // 2] - math.cos(1.0)) < 1e-15
    assert np.count_nonzero(np.abs(y) > 1e-15) == 2


# ---- attention ----------------------------------------------------------------------------------

def test_attention_single_key_returns_its_value():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((3, 64))
    k = rng.standard_normal((1, 64))
    v = rng.standard_normal((1, 64))
    assert np.allclose(od.attention(q, k, v), np.repeat(v, 3, 0), atol=1e-15)


def test_attention_identical_keys_average_values():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((4, 32))
    k = np.repeat(rng.standard_normal((1, 32)), 9, 0)
    v = rng.standard_normal((9, 32))
    assert np.allclose(od.attention(q, k, v), np.repeat(v.mean(0, keepdims=True), 4, 0),
                       atol=1e-14)


def test_attention_matches_explicit_loops():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((3, 8))
    k = rng.standard_normal((5, 8)) * 3
    v = rng.standard_normal((5, 8))
    out = np.zeros((3, 8))
    for i in range(3):
        s = [sum(q[i, d] * k[j, d] for d in range(8)) / math.sqrt(8) for j in range(5)]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        tot = sum(e)
        for j in range(5):
            out[i] += e[j] / tot * v[j]
    assert np.allclose(od.attention(q, k, v), out, atol=1e-14)


# ---- the composed forward: structure the pages fix ----------------------------------------------

def _fwd(W, toks, h, **kw):
    return od.drafter_forward(TINY, W, toks, 1, hidden=h, **kw)


def test_block_attention_is_bidirectional(tiny_w):
    """Changing a later block token changes the outputs of earlier mask positions."""
    h = _hidden(64)
    toks = [5] + [TINY.mask_token_id] * 7
    a = _fwd(tiny_w, toks, h)["logits"]
    toks2 = list(toks)
    toks2[6] = 17
    b = _fwd(tiny_w, toks2, h)["logits"]
    assert np.max(np.abs(a[0] - b[0])) > 1e-6       # row 0 = block position 1 sees position 6


def test_every_block_output_reaches_every_context_position(tiny_w):
    h = _hidden(64)
    toks = [5] + [TINY.mask_token_id] * 7
    a = _fwd(tiny_w, toks, h)["logits"]
    for p in (0, 31, 63):
        h2 = h.copy()
        h2[p] += 1.0
        b = _fwd(tiny_w, toks, h2)["logits"]
        assert np.all(np.max(np.abs(a - b), axis=1) > 1e-8)


def test_mask_rows_differ(tiny_w):
    """Positions make the identical [MASK] inputs produce different outputs."""
    h = _hidden(64)
    lg = _fwd(tiny_w, [5] + [TINY.mask_token_id] * 7, h)["logits"]
    for i in range(1, lg.shape[0]):
        assert np.max(np.abs(lg[i] - lg[0])) > 1e-6


def test_incremental_ingest_equals_cold(tiny_w):
    h = _hidden(64)
    for l in range(TINY.n_layers):
        k64, v64 = od.context_kv(TINY, tiny_w, l, h)
        k56, v56 = od.context_kv(TINY, tiny_w, l, h[:56])
        k8, v8 = od.context_kv(TINY, tiny_w, l, h[56:], pos0=56)
        assert np.allclose(np.concatenate([k56, k8], 1), k64, atol=1e-13, rtol=0)
        assert np.allclose(np.concatenate([v56, v8], 1), v64, atol=1e-13, rtol=0)
    toks = [9] + [TINY.mask_token_id] * 7
    cold = _fwd(tiny_w, toks, h)
    warm = od.drafter_forward(TINY, tiny_w, toks, 1, ctx_kv=cold["ctx_kv"])
    assert np.array_equal(cold["logits"], warm["logits"])


def test_shared_kv_projection_equals_one_projection_over_both_sources(tiny_w):
    """With W_kc = W_kd and W_vc = W_vd (the 'no KV split' ablation on the DFlare page), one
    layer's attention equals a single K/V projection of [context features; block features],
    written out here with explicit per-head loops."""
    W = dict(tiny_w)
    W["wk_ctx"], W["wv_ctx"] = W["wk_draft"], W["wv_draft"]
    one = TINY.__class__(**{**TINY.__dict__, "n_layers": 1})
    W1 = {k: (v[:1] if k not in ("embed", "lm_head", "final_norm_w") else v) for k, v in
          W.items()}
    h = _hidden(12)
    toks = [3] + [one.mask_token_id] * 7
    out = od.drafter_forward(one, W1, toks, 1, hidden=h, keep=True)["resid"][0]
    # independent recomputation of layer 0's attention block output
    c = od.context_features(one, W1, 0, h)
    x = W1["embed"][toks].astype(np.float64)
    xn = od.rmsnorm(x, W1["attn_norm_w"][0], one.rms_eps)
    feats = np.concatenate([c, xn], 0)                                    # [12 + 8, H]
    pos = np.arange(20)
    K = od.rope((feats @ W1["wk_draft"][0].T.astype(np.float64)).reshape(20, 2, 64), pos, 1e6)
    Vv = (feats @ W1["wv_draft"][0].T.astype(np.float64)).reshape(20, 2, 64)
    Q = od.rope((xn @ W1["wq"][0].T.astype(np.float64)).reshape(8, 4, 64), pos[12:], 1e6)
    o = np.zeros((8, 4, 64))
    for hh in range(4):
        g = hh // 2
        for i in range(8):
            s = np.array([np.dot(Q[i, hh], K[j, g]) for j in range(20)]) / 8.0
            e = np.exp(s - s.max())
            o[i, hh] = (e / e.sum()) @ Vv[:, g]
    x = x + o.reshape(8, 256) @ W1["wo"][0].T.astype(np.float64)
    xm = od.rmsnorm(x, W1["mlp_norm_w"][0], one.rms_eps)
    gt = xm @ W1["w_gate"][0].T.astype(np.float64)
    up = xm @ W1["w_up"][0].T.astype(np.float64)
    x = x + (gt / (1 + np.exp(-gt)) * up) @ W1["w_down"][0].T.astype(np.float64)
    assert np.max(np.abs(out - x)) < 1e-12


def test_silu_closed_form():
    z = np.array([0.0, 1.0, -1.0, 40.0, -40.0])
    s = od.silu(z)
    assert s[0] == 0.0
    assert abs(s[1] - 1 / (1 + math.exp(-1))) < 1e-16
    assert abs(s[2] + 1 / (1 + math.e)) < 1e-16
    assert abs(s[3] - 40.0) < 1e-12 and abs(s[4]) < 1e-15


def test_logits_cover_mask_rows_only(tiny_w):
    lg = _fwd(tiny_w, [5] + [TINY.mask_token_id] * 7, _hidden(64))["logits"]
    assert lg.shape == (7, TINY.vocab)


def _planted_final_gain():
    """A final-norm gain far from 1 and different in every element."""
    return 0.25 + 1.5 * np.arange(TINY.hidden, dtype=np.float64) / TINY.hidden


def test_lm_head_with_silent_layers_is_the_normed_embedding_by_hand(tiny_w):
    """With W_o = W_down = 0 every layer adds zero, so the final residual is the block's
    embedding.  Logits row j must then be RMSNorm(E[block token n_anchor + j]) * g_fin times the
    LM head, written here as explicit sums over the hidden dimension for a few vocab entries.
    The anchor's embedding differs from the mask's, so taking rows 0..D-1 instead of the mask rows
    fails, and so does a dropped or uniform gain."""
    W = dict(tiny_w)
    W["wo"] = np.zeros_like(W["wo"])
    W["w_down"] = np.zeros_like(W["w_down"])
    g = _planted_final_gain()
    W["final_norm_w"] = g
    toks = [5] + [TINY.mask_token_id] * 7
    lg = _fwd(W, toks, _hidden(16))["logits"]
    H, eps = TINY.hidden, TINY.rms_eps
    E, Wlm = W["embed"], W["lm_head"]
    for j in range(len(toks) - 1):
        e = [float(v) for v in E[toks[1 + j]]]
        r = 1.0 / math.sqrt(sum(v * v for v in e) / H + eps)
        for vtok in (0, 1, 77, TINY.vocab - 2, TINY.vocab - 1):
            ref = sum(e[h] * r * g[h] * float(Wlm[vtok, h]) for h in range(H))
            assert abs(lg[j, vtok] - ref) < 1e-12 * max(1.0, abs(ref)), (j, vtok)
    # the anchor row's value is different, so the rows really are the mask rows
    e0 = E[toks[0]].astype(np.float64)
    a0 = (e0 / np.sqrt(np.mean(e0 * e0) + eps) * g) @ Wlm.T.astype(np.float64)
    assert np.max(np.abs(a0 - lg[0])) > 1e-3


def test_lm_head_rows_are_the_final_mask_residuals(tiny_w):
    """Identity LM head (V = H) and a planted gain: logits row j equals RMSNorm(final residual
    row n_anchor + j) * g_fin element by element (the residual from the forward's own per-layer
    record), and differs from the anchor row's normed residual."""
    sh = TINY.__class__(**{**TINY.__dict__, "vocab": TINY.hidden})
    W = dict(tiny_w)
    W["embed"] = tiny_w["embed"][:TINY.hidden]
    W["lm_head"] = np.eye(TINY.hidden)
    g = _planted_final_gain()
    W["final_norm_w"] = g
    toks = [5] + [sh.vocab - 1] * 7
    out = od.drafter_forward(sh, W, toks, 1, hidden=_hidden(20), keep=True)
    x = out["resid"][-1]
    H, eps = sh.hidden, sh.rms_eps
    for j in range(len(toks) - 1):
        row = x[1 + j]
        r = 1.0 / math.sqrt(sum(float(v) * float(v) for v in row) / H + eps)
        ref = np.array([row[h] * r * g[h] for h in range(H)])
        assert np.max(np.abs(out["logits"][j] - ref)) < 1e-12
    a = x[0] / math.sqrt(float(np.mean(x[0] * x[0])) + eps) * g
    assert np.max(np.abs(out["logits"][0] - a)) > 1e-3
    # with no anchor every row is a mask row: D = B
    out0 = od.drafter_forward(sh, W, toks, 0, hidden=_hidden(20), keep=True)
    assert out0["logits"].shape == (8, H)
    x0 = out0["resid"][-1]
    assert np.max(np.abs(out0["logits"][0] - x0[0] / math.sqrt(float(np.mean(x0[0] ** 2)) + eps)
                         * g)) < 1e-12


# ---- the workload shapes follow the pages' stated structure -------------------------------------

def test_workloads_follow_page_constants():
    g = json.load(open(os.path.join(GOLDEN, "page_constants.json")))
    for name in ("qwen3-4b", "qwen3-8b"):
        wl = synth.workload(name)
        assert (wl.shape.n_layers, wl.block_len, wl.shape.n_target_layers) == (
            g["dflare_qwen"]["draft_layers"], g["dflare_qwen"]["block_len"],
            g["dflare_qwen"]["target_layers"])
        assert wl.shape.n_layers * wl.shape.n_target_layers == \
            g["dflare_mix_coefficients_7x9"]["value"]
    wl = synth.workload("gpt-oss-20b")
    assert (wl.shape.n_layers, wl.block_len, wl.shape.n_target_layers) == (
        g["dflare_gpt_oss"]["draft_layers"], g["dflare_gpt_oss"]["block_len"],
        g["dflare_gpt_oss"]["target_layers"])
    wl = synth.workload("specdiff2-7b")
    assert wl.block_len == g["specdiff2_window"]["diffucoder_gamma"] and wl.n_anchor == 0
    assert wl.n_drafts <= g["specdiff2_selection_K_T"]["K_max"]
    assert wl.temperature in g["specdiff2_selection_K_T"]["temperatures"]
    # planted per-position rates reproduce the pages' acceptance lengths
    for name, tau in g["dflare_accept_len_T0"].items():
        if name == "cite":
            continue
        wl = synth.workload(name)
        a = wl.planted_alpha
        assert abs(1 + sum(a ** m for m in range(1, wl.n_draft + 1)) - tau) < 0.01
    # reading: the reported streak, like the acceptance length, counts the verifier's own token
    wl = synth.workload("specdiff2-7b")
    a = wl.planted_alpha
    assert abs(1 + sum(a ** m for m in range(1, 33)) - g["specdiff2_avg_streak"]["value"]) < 0.01


# ---- context-path variants: fully connected fusion, raw mixing, shared K/V ---------------------

TINY_FC = synth.workload("tiny-dflash-fp32").shape
TINY_ABL = synth.workload("tiny-ablate-fp32").shape


def test_fc_fusion_with_block_scalar_weights_equals_mixing(tiny_w):
    """W_fc = [w_0 I | w_1 I | ...] with w the softmax mixing coefficients of a layer, and the same
    gain, makes the fully connected fusion the same weighted sum as that layer's mixing."""
    H, Lt = TINY.hidden, TINY.n_target_layers
    h = _hidden(9)
    for l in range(TINY.n_layers):
        w = od.mix_weights(tiny_w["mix_logits"])[l]
        Wfc = {"fc_w": np.concatenate([w[i] * np.eye(H) for i in range(Lt)], axis=1),
               "fc_norm_w": tiny_w["mix_norm_w"][l]}
        a = od.context_features(TINY_FC, Wfc, l, h)
        b = od.context_features(TINY, tiny_w, l, h)
        assert np.max(np.abs(a - b)) < 1e-12


def test_fc_fusion_concatenates_target_layers_in_order():
    """A fully connected layer that reads only target layer i's block of the concatenation
    (identity there, zero elsewhere) gives RMSNorm(h_i) * g for every draft layer."""
    H, Lt = TINY.hidden, TINY.n_target_layers
    h = _hidden(7)
    g = 1.0 + 0.1 * np.arange(H) / H
    for i in range(Lt):
        fc = np.zeros((H, Lt * H))
        fc[:, i * H:(i + 1) * H] = np.eye(H)
        c = od.context_features(TINY_FC, {"fc_w": fc, "fc_norm_w": g}, 1, h)
        ref = h[:, i, :] / np.sqrt(np.mean(h[:, i, :].astype(np.float64) ** 2, 1, keepdims=True)
                                   + TINY.rms_eps) * g
        assert np.max(np.abs(c - ref)) < 1e-12


def test_raw_mixing_with_log_coefficients_equals_softmax_mixing(tiny_w):
    """Without softmax the coefficients are used as given: coefficients w that sum to 1 give the
    same features as softmax mixing over logits log(w)."""
    h = _hidden(6)
    rng = np.random.default_rng(3)
    w = rng.dirichlet(np.ones(TINY.n_target_layers), size=TINY.n_layers)
    Wraw = dict(tiny_w, mix_logits=w)
    Wsm = dict(tiny_w, mix_logits=np.log(w))
    for l in range(TINY.n_layers):
        a = od.context_features(TINY_ABL, Wraw, l, h)
        b = od.context_features(TINY, Wsm, l, h)
        assert np.max(np.abs(a - b)) < 1e-12


def test_raw_mixing_is_linear_in_the_coefficients(tiny_w):
    """Raw coefficients a and 3a give the same features up to RMSNorm's epsilon (the norm removes
    the scale), while softmax(a) and softmax(3a) differ."""
    h = _hidden(5)
    W1 = dict(tiny_w)
    W3 = dict(tiny_w, mix_logits=3.0 * tiny_w["mix_logits"])
    a = od.context_features(TINY_ABL, W1, 0, h)
    b = od.context_features(TINY_ABL, W3, 0, h)
    assert np.max(np.abs(a - b)) < 1e-5
    assert np.max(np.abs(od.context_features(TINY, W1, 0, h) -
                         od.context_features(TINY, W3, 0, h))) > 1e-2


def test_shared_kv_switch_uses_the_draft_projection(tiny_w):
    """Context K/V without the split equal the split path with W_kc := W_kd, W_vc := W_vd."""
    h = _hidden(10)
    W = dict(tiny_w)
    W["wk_ctx"], W["wv_ctx"] = W["wk_draft"], W["wv_draft"]
    shared = TINY.__class__(**{**TINY.__dict__, "ctx_shared_kv": True})
    for l in range(TINY.n_layers):
        k1, v1 = od.context_kv(shared, tiny_w, l, h, pos0=3)
        k2, v2 = od.context_kv(TINY, W, l, h, pos0=3)
        assert np.array_equal(k1, k2) and np.array_equal(v1, v2)


def test_generated_weights_follow_the_context_path():
    fc = synth.make_weights(TINY_FC, seed=0)
    abl = synth.make_weights(TINY_ABL, seed=0)
    H, Lt = TINY.hidden, TINY.n_target_layers
    assert tuple(fc["fc_w"].shape) == (H, Lt * H) and "mix_logits" not in fc
    assert "wk_ctx" not in fc and "wk_ctx" not in abl and "mix_logits" in abl
