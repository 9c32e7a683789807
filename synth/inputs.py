"""Seeded synthetic tensors for the workloads in ``configs``.

Every tensor is drawn from its own ``torch.Generator`` on the requested device, seeded from
(workload seed, tensor name), so a tensor does not depend on which other tensors were drawn.  The
same seed gives different values on CPU and GPU (the generators differ); a test that compares two
implementations generates once and hands the same tensor to both.

Distributions (the configurations' own statement): linear, embedding and LM-head weights
N(0, 0.02); norm gains 1 + N(0, 0.02) so that a missing gain multiply shows; mixing logits N(0, 1);
target hidden states N(0, 1); verify logits N(0, std) fp32.  bf16 tensors are fp32 draws rounded
to nearest-even by ``Tensor.to``.
"""
import zlib

import numpy as np
import torch

from .configs import DrafterShape, Workload

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def tensor_seed(seed: int, name: str) -> int:
    """A stable 63-bit seed for one named tensor."""
    return ((int(seed) * 1_000_003) ^ (zlib.crc32(name.encode()) << 20)) & ((1 << 63) - 1)


def _gen(device, seed: int, name: str) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(tensor_seed(seed, name))
    return g


def _randn(shape, device, seed, name, std=1.0, mean=0.0, dtype=torch.float32):
    g = _gen(device, seed, name)
    t = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    if mean != 0.0:
        t.add_(mean)
    return t.to(dtype)


def make_weights(shape: DrafterShape, seed: int = 0, device="cpu") -> dict:
    """Drafter weights, Linear layout [out, in] row-major, stacked over draft layers."""
    dt = _DT[shape.dtype]
    L, H, F, V = shape.n_layers, shape.hidden, shape.ffn, shape.vocab
    qd, kd = shape.q_dim, shape.kv_dim
    w = {}

    def lin(name, *s):
        w[name] = _randn(s, device, seed, name, std=0.02, dtype=dt)

    def gain(name, *s):
        w[name] = _randn(s, device, seed, name, std=0.02, mean=1.0, dtype=dt)

    if shape.n_target_layers > 0:
        if shape.ctx_fusion == "fc":
            lin("fc_w", H, shape.n_target_layers * H)
            gain("fc_norm_w", H)
        else:
            w["mix_logits"] = _randn((L, shape.n_target_layers), device, seed, "mix_logits")
            gain("mix_norm_w", L, H)
        if not shape.ctx_shared_kv:
            lin("wk_ctx", L, kd, H)
            lin("wv_ctx", L, kd, H)
    gain("attn_norm_w", L, H)
    gain("mlp_norm_w", L, H)
    lin("wq", L, qd, H)
    lin("wk_draft", L, kd, H)
    lin("wv_draft", L, kd, H)
    lin("wo", L, H, qd)
    lin("w_gate", L, F, H)
    lin("w_up", L, F, H)
    lin("w_down", L, H, F)
    gain("final_norm_w", H)
    lin("embed", V, H)
    lin("lm_head", V, H)
    return w


def leading_successes(rng: np.random.Generator, alpha: float, cap: int) -> int:
    """Number of leading successes of Bernoulli(alpha) trials, at most ``cap``."""
    n = 0
    while n < cap and rng.random() < alpha:
        n += 1
    return n


def make_lengths(wl: Workload, seed: int = 0):
    """Per-sequence cached context length and number of newly committed positions to ingest.

    Cached lengths are uniform integers in [ctx_lo, ctx_hi]; the new-position count is one plus
    the planted leading successes (what the previous verify committed), unless fixed."""
    rng = np.random.default_rng(tensor_seed(seed, "lengths"))
    ctx = rng.integers(wl.ctx_lo, wl.ctx_hi + 1, size=wl.batch).astype(np.int64)
    if wl.fixed_new >= 0:
        new = np.full(wl.batch, wl.fixed_new, dtype=np.int64)
    else:
        new = np.array([1 + leading_successes(rng, wl.planted_alpha, wl.n_draft)
                        for _ in range(wl.batch)], dtype=np.int64)
    return ctx, new


def capacity_for(wl: Workload, ctx, new, align: int = 64) -> int:
    need = int(np.max(np.asarray(ctx) + np.asarray(new))) + wl.block_len
    return (need + align - 1) // align * align


def make_block_tokens(wl: Workload, seed: int = 0, device="cpu") -> torch.Tensor:
    """[N, B] int32: anchor (a random non-mask token) followed by [MASK] ids; all masks if no
    anchor."""
    V = wl.shape.vocab
    g = _gen(device, seed, "block_tokens")
    t = torch.full((wl.batch, wl.block_len), wl.shape.mask_token_id, dtype=torch.int32,
                   device=device)
    if wl.n_anchor:
        t[:, : wl.n_anchor] = torch.randint(0, V - 1, (wl.batch, wl.n_anchor), generator=g,
                                            device=device, dtype=torch.int32)
    return t


def make_hidden(shape: DrafterShape, n_tokens: int, seed: int, seq: int, device="cpu",
                start: int = 0) -> torch.Tensor:
    """Target hidden states of sequence ``seq`` for positions [start, start + n_tokens):
    [n_tokens, L_t, H] in the model dtype.  Position p of a sequence always gets the same
    values, whatever ``start`` is (one draw per position block of 64)."""
    dt = _DT[shape.dtype]
    Lt, H = shape.n_target_layers, shape.hidden
    out = torch.empty((n_tokens, Lt, H), dtype=dt, device=device)
    blk = 64
    p = start
    while p < start + n_tokens:
        b0 = p // blk * blk
        chunk = _randn((blk, Lt, H), device, seed, f"hidden/{seq}/{b0}", dtype=dt)
        lo, hi = p - b0, min(blk, start + n_tokens - b0)
        out[p - start: p - start + (hi - lo)] = chunk[lo:hi]
        p += hi - lo
    return out


def make_cache_kv(shape: DrafterShape, batch: int, ctx_len: int, seed: int = 0, device="cpu"):
    """Synthetic post-RoPE context K and V for a drafter that takes its context from a cache:
    two tensors [L, N, kvh, ctx_len, hd], N(0, 1), model dtype."""
    dt = _DT[shape.dtype]
    s = (shape.n_layers, batch, shape.n_kv_heads, ctx_len, shape.head_dim)
    return (_randn(s, device, seed, "cache_k", dtype=dt),
            _randn(s, device, seed, "cache_v", dtype=dt))


def make_drafts(batch: int, n_drafts: int, n_draft: int, vocab: int, seed: int = 0,
                device="cpu", name="drafts") -> torch.Tensor:
    """[N, K, D] int32 uniform random tokens (mask id excluded)."""
    g = _gen(device, seed, name)
    return torch.randint(0, vocab - 1, (batch, n_drafts, n_draft), generator=g, device=device,
                         dtype=torch.int32)


def make_planted_verify_logits(drafts: torch.Tensor, n_rows: int, vocab: int, alpha: float,
                               std: float = 2.0, seed: int = 0, device="cpu"):
    """Target logits [N, R, V] fp32 N(0, std) with a planted accepted-prefix length per sequence.

    drafts: [N, D].  For sequence n a length a_n (leading Bernoulli(alpha) successes, at most D) is
    drawn; rows j < a_n get the draft token's logit set one above the row's largest value, and row
    a_n, if it exists and its largest value sits at the draft token, gets that logit set one below
    the row's smallest value.  Returns (logits, a) with a the planted lengths as a numpy array."""
    N, D = drafts.shape
    logits = _randn((N, n_rows, vocab), device, seed, "verify_logits", std=std)
    rng = np.random.default_rng(tensor_seed(seed, "verify_plant"))
    a = np.array([leading_successes(rng, alpha, D) for _ in range(N)], dtype=np.int64)
    d = drafts.to("cpu").numpy()
    for n in range(N):
        for j in range(min(int(a[n]), n_rows)):
            row = logits[n, j]
            row[int(d[n, j])] = row.max() + 1.0
        j = int(a[n])
        if j < D and j < n_rows:
            row = logits[n, j]
            tok = int(d[n, j])
            if float(row[tok]) >= float(row.max()):
                row[tok] = row.min() - 1.0
    return logits, a


def make_planted_streak_logits(drafts: torch.Tensor, n_rows: int, vocab: int, alpha: float,
                               std: float = 2.0, seed: int = 0, device="cpu"):
    """Verifier logits [N, K, R, V] fp32 for K drafts per sequence, planted per (n, k) as in
    ``make_planted_verify_logits`` but with the draft token raised by a random margin
    delta ~ U[0, 6] above the row's largest value, so that streak scores spread out.

    drafts: [N, K, G].  Returns (logits, a) with a [N, K]."""
    N, K, G = drafts.shape
    logits = _randn((N, K, n_rows, vocab), device, seed, "streak_logits", std=std)
    rng = np.random.default_rng(tensor_seed(seed, "streak_plant"))
    a = np.zeros((N, K), dtype=np.int64)
    d = drafts.to("cpu").numpy()
    for n in range(N):
        for k in range(K):
            a[n, k] = leading_successes(rng, alpha, G)
            for j in range(min(int(a[n, k]), n_rows)):
                row = logits[n, k, j]
                row[int(d[n, k, j])] = row.max() + float(rng.uniform(0.0, 6.0))
            j = int(a[n, k])
            if j < G and j < n_rows:
                row = logits[n, k, j]
                tok = int(d[n, k, j])
                if float(row[tok]) >= float(row.max()):
                    row[tok] = row.min() - 1.0
    return logits, a
