"""Block-diffusion drafter forward pass: the slow, plain fp64 CPU definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix (DFlare page, sections on parallel drafting, on per-draft-layer mixing and on
splitting K/V projections by source; DFlash article, section on writing a whole block in one
forward pass; SpecDiff-2 notes, section 4):
* one forward pass predicts every mask position of a block [anchor, MASK, ..., MASK];
* attention inside the block is bidirectional and the block reaches the whole context;
* each draft layer mixes several target hidden layers with its own softmax-normalised weights,
  then applies RMSNorm;
* target-context features and draft-block features get separate K and V projections; queries come
  from the draft features; target cues enter the K/V of every draft layer;
* the embedding and LM head are shared and frozen.

Readings where the pages are silent (each listed with its reason in the design notes): a
pre-norm decoder layer with a SwiGLU MLP and no biases; RMSNorm y = x / sqrt(mean(x^2) + eps) * g;
rotate-half RoPE on queries and on both kinds of keys, context positions 0..C-1 and block
positions C..C+B-1; the LM head runs over the mask rows only; a drafter without target mixing
(n_target_layers = 0) takes its context K/V, already rotated, from a cache.

Every real-valued step is fp64 from the exact stored inputs.  The function is stateless: the
context K/V are recomputed from all context hidden states unless given.
"""
import numpy as np


def f64(a) -> np.ndarray:
    """Exact upcast of a numpy array or a CPU torch tensor (fp32/bf16) to fp64."""
    if hasattr(a, "detach"):                      # torch tensor
        a = a.detach().to("cpu")
        if str(a.dtype) == "torch.bfloat16":
            a = a.float()
        a = a.numpy()
    return np.asarray(a, dtype=np.float64)


def softmax_rows(a) -> np.ndarray:
    a = np.asarray(a, np.float64)
    z = a - a.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def rmsnorm(x, g, eps: float) -> np.ndarray:
    """y = x / sqrt(mean(x^2) + eps) * g over the last axis."""
    x = np.asarray(x, np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(g, np.float64)


def silu(z) -> np.ndarray:
    z = np.asarray(z, np.float64)
    return z / (1.0 + np.exp(-z))


def rope(x, pos, theta: float) -> np.ndarray:
    """Rotate-half rotary embedding.  x: [T, heads, hd]; pos: [T] integer positions.
    Pair (d, d + hd/2) is rotated by the angle pos * theta^(-2d/hd)."""
    x = np.asarray(x, np.float64)
    hd = x.shape[-1]
    half = hd // 2
    inv_freq = theta ** (-(2.0 * np.arange(half, dtype=np.float64)) / hd)
    ang = np.asarray(pos, np.float64)[:, None] * inv_freq[None, :]          # [T, half]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def mix_weights(mix_logits, raw: bool = False) -> np.ndarray:
    """Mixing coefficients, one row per draft layer: [L_d, L_t].  Softmax over the target layers
    (DFlare page, per-layer mixing section), or the given values as they are (raw = True: the
    page's "without softmax" ablation)."""
    return f64(mix_logits) if raw else softmax_rows(f64(mix_logits))


def context_features(shape, W, layer: int, hidden) -> np.ndarray:
    """Context features of draft layer `layer` from target hidden states [T, L_t, H] -> [T, H].

    Mixing (DFlare page, per-layer mixing section): c_l(t) = RMSNorm(sum_i w_{l,i} h_i(t)) *
    g_mix_l with w the mixing coefficients of the layer.
    Fully connected fusion (DFlare page, comparison with DFlash; DFlash article, section on
    conditioning every layer on target features): one shared feature for every draft layer,
    c(t) = RMSNorm(W_fc . [h_0(t); h_1(t); ...; h_{L_t-1}(t)]) * g_fc, the target layers
    concatenated in order; the RMSNorm after the fusion is a reading (the pages name only the
    fully connected layer), matching the normalisation of the mixing path."""
    h = f64(hidden)
    if getattr(shape, "ctx_fusion", "mix") == "fc":
        T = h.shape[0]
        m = h.reshape(T, -1) @ f64(W["fc_w"]).T
        return rmsnorm(m, f64(W["fc_norm_w"]), shape.rms_eps)
    w = mix_weights(W["mix_logits"], getattr(shape, "mix_raw", False))[layer]     # [L_t]
    m = np.einsum("i,tih->th", w, h)
    return rmsnorm(m, f64(W["mix_norm_w"][layer]), shape.rms_eps)


def context_projection(shape, W, layer: int):
    """The (K, V) weights that project context features: the context's own (DFlare page, section
    on splitting the K/V projections by source) or, without the split, the draft block's."""
    if getattr(shape, "ctx_shared_kv", False):
        return W["wk_draft"][layer], W["wv_draft"][layer]
    return W["wk_ctx"][layer], W["wv_ctx"][layer]


def context_kv(shape, W, layer: int, hidden, pos0: int = 0):
    """Context K (rotated) and V of one draft layer from target hidden states of positions
    pos0 .. pos0+T-1: two arrays [kvh, T, hd]."""
    c = context_features(shape, W, layer, hidden)
    T = c.shape[0]
    kvh, hd = shape.n_kv_heads, shape.head_dim
    wk, wv = context_projection(shape, W, layer)
    k = (c @ f64(wk).T).reshape(T, kvh, hd)
    v = (c @ f64(wv).T).reshape(T, kvh, hd)
    k = rope(k, np.arange(pos0, pos0 + T), shape.rope_theta)
    return k.transpose(1, 0, 2), v.transpose(1, 0, 2)


def attention(q, k, v) -> np.ndarray:
    """softmax(q k^T / sqrt(hd)) v with no mask.  q: [Tq, hd]; k, v: [Tk, hd]."""
    s = (q @ k.T) / np.sqrt(q.shape[-1])
    return softmax_rows(s) @ v


def drafter_forward(shape, W, block_tokens, n_anchor: int, hidden=None, ctx_kv=None,
                    keep=False):
    """One drafter forward pass for one sequence.

    block_tokens: [B] token ids (anchor then masks).
    hidden: [C, L_t, H] target hidden states of every context position (cold recompute), or
    ctx_kv: per layer (K [kvh, C, hd] rotated, V [kvh, C, hd]).
    Returns a dict: logits [D, V] fp64, ctx_kv, and (keep=True) per-layer residuals.
    """
    L, H = shape.n_layers, shape.hidden
    qh, kvh, hd = shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    grp = qh // kvh
    if ctx_kv is None:
        C = f64(hidden).shape[0] if hidden is not None else 0
        ctx_kv = [context_kv(shape, W, l, hidden) for l in range(L)]
    C = ctx_kv[0][0].shape[1]
    toks = np.asarray(block_tokens, dtype=np.int64)
    B = toks.shape[0]
    pos = np.arange(C, C + B)
    E = W["embed"]
    x = np.stack([f64(E[int(t)]) for t in toks])                              # [B, H]
    resid = []
    for l in range(L):
        xn = rmsnorm(x, f64(W["attn_norm_w"][l]), shape.rms_eps)
        q = rope((xn @ f64(W["wq"][l]).T).reshape(B, qh, hd), pos, shape.rope_theta)
        kd = rope((xn @ f64(W["wk_draft"][l]).T).reshape(B, kvh, hd), pos, shape.rope_theta)
        vd = (xn @ f64(W["wv_draft"][l]).T).reshape(B, kvh, hd)
        kc, vc = ctx_kv[l]
        o = np.zeros((B, qh, hd))
        for h in range(qh):
            g = h // grp
            kk = np.concatenate([f64(kc[g]), kd[:, g, :]], axis=0)
            vv = np.concatenate([f64(vc[g]), vd[:, g, :]], axis=0)
            o[:, h, :] = attention(q[:, h, :], kk, vv)
        x = x + o.reshape(B, qh * hd) @ f64(W["wo"][l]).T
        xm = rmsnorm(x, f64(W["mlp_norm_w"][l]), shape.rms_eps)
        gate = xm @ f64(W["w_gate"][l]).T
        up = xm @ f64(W["w_up"][l]).T
        x = x + (silu(gate) * up) @ f64(W["w_down"][l]).T
        if keep:
            resid.append(x.copy())
    xf = rmsnorm(x[n_anchor:], f64(W["final_norm_w"]), shape.rms_eps)
    logits = xf @ f64(W["lm_head"]).T
    return {"logits": logits, "ctx_kv": ctx_kv, "resid": resid}
