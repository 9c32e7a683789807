"""Build one synthetic workload on the GPU, run the library on it, and prepare the oracle's view
of the same inputs.  Shared by the GPU parity tests (not collected itself)."""
from dataclasses import replace

import numpy as np
import torch

import block_diffusion_drafter_draft_amd as dbd
import synth

DT = {"f32": torch.float32, "bf16": torch.bfloat16}


class Case:
    """Inputs of one draft_block step for workload ``wl`` plus the library's outputs.

    The cache holds the cached context of every sequence: filled by a cold draft_block call that
    ingests positions 0 .. C_n-1 (target-mixing drafters) or copied from synthetic rotated K/V
    (drafters that take their context from a cache).  The measured step then ingests n_new
    positions and drafts the block."""

    def __init__(self, wl, seed=0, dev="cuda", ctx=None, new=None, seqs_hidden=None):
        self.wl, self.dev, self.seed = wl, dev, seed
        self._oracle_w = None
        self.last_ws = None
        sh = wl.shape
        self.shape = sh
        self.desc = dbd.model_desc(sh, act_pairs=wl.act_pairs)
        self.W = synth.make_weights(sh, seed, dev)
        self.wstruct = dbd.weights_struct(self.W)
        c, n = synth.make_lengths(wl, seed)
        self.ctx = np.asarray(ctx if ctx is not None else c, np.int64)
        self.new = np.asarray(new if new is not None else n, np.int64)
        self.cap = synth.capacity_for(wl, self.ctx, self.new)
        N, B = wl.batch, wl.block_len
        self.tokens = synth.make_block_tokens(wl, seed, dev)
        L, kvh, hd = sh.n_layers, sh.n_kv_heads, sh.head_dim
        dt = DT[sh.dtype]
        ks, vs = dbd.kv_cache_shapes(sh, N, self.cap)
        self.kv_k = torch.zeros(ks, dtype=dt, device=dev)
        self.kv_v = torch.zeros(vs, dtype=dt, device=dev)
        self.D = B - wl.n_anchor
        self.cache_kv = None
        if wl.ctx_source == "hidden":
            self.hidden = [synth.make_hidden(sh, int(self.ctx[i] + self.new[i]), seed, i, dev)
                           for i in range(N)]
        else:
            K, V = synth.make_cache_kv(sh, N, int(self.ctx.max()), seed, dev)
            self.cache_kv = (K, V)
            for i in range(N):
                C = int(self.ctx[i])
                C8 = (C + 7) // 8 * 8
                self.kv_k[:, i, :, :C, :] = K[:, i, :, :C, :]
                vpad = torch.zeros((L, kvh, C8, hd), dtype=dt, device=dev)
                vpad[:, :, :C] = V[:, i, :, :C, :]
                self.kv_v[:, i, :, : C8 // 8] = dbd.pack_values(vpad)

    # ------------------------------------------------------------------ running the library
    def _offsets(self, counts):
        off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        return torch.tensor(off, device=self.dev), int(off[-1])

    def _hidden_rows(self, lo, hi):
        rows = [self.hidden[i][int(lo[i]):int(hi[i])] for i in range(self.wl.batch)]
        return torch.cat(rows, 0).contiguous()

    def workspace(self, n_new_total, n_drafts, temperature, desc=None):
        nb = dbd.draft_workspace_bytes(desc or self.desc, self.wl.batch, self.wl.block_len,
                                       self.wl.n_anchor, n_new_total, n_drafts, temperature,
                                       self.cap)
        return torch.empty(nb, dtype=torch.uint8, device=self.dev)

    def call(self, ctx_len, counts, hidden, n_drafts=None, temperature=None, seed=1234,
             logits=True, desc=None):
        wl = self.wl
        desc = desc or self.desc
        K = n_drafts if n_drafts is not None else wl.n_drafts
        T = temperature if temperature is not None else wl.temperature
        off, tot = self._offsets(counts)
        ws = self.workspace(tot, K, T, desc)
        self.last_ws = ws
        out = torch.full((wl.batch, K, self.D), -7, dtype=torch.int32, device=self.dev)
        lg = (torch.empty((wl.batch, self.D, self.shape.vocab), dtype=torch.float32,
                          device=self.dev) if logits else None)
        st = torch.full((wl.batch,), -7, dtype=torch.int32, device=self.dev)
        dbd.draft_block(desc, self.wstruct, self.tokens, hidden, off,
                        torch.tensor(np.asarray(ctx_len, np.int32), device=self.dev), self.kv_k,
                        self.kv_v, out, ws, tot, n_drafts=K, temperature=T, seed=seed,
                        n_anchor=wl.n_anchor, logits_out=lg, seq_status=st)
        return out, lg, st

    def fill_cache(self):
        """Cold ingest of positions 0 .. C_n-1 (target-mixing drafters only)."""
        if self.wl.ctx_source != "hidden":
            return
        zeros = np.zeros(self.wl.batch, np.int64)
        h = self._hidden_rows(zeros, self.ctx)
        self.call(zeros, self.ctx, h if h.numel() else None, logits=False)

    def step(self, **kw):
        """The measured step: ingest n_new positions at C_n, draft the block."""
        if self.wl.ctx_source == "hidden":
            h = self._hidden_rows(self.ctx, self.ctx + self.new)
            return self.call(self.ctx, self.new, h if h.numel() else None, **kw)
        return self.call(self.ctx, np.zeros(self.wl.batch, np.int64), None, **kw)

    def residuals(self):
        """The block's fp32 residual stream after every draft layer, [L][N, B, H] numpy, from
        calls of the measured step with the drafter truncated to l + 1 layers (the stacked
        weights and cache layers of the first l + 1 layers are prefixes of the full ones, so
        the call recomputes exactly the full step's first l + 1 layers)."""
        sh, wl = self.shape, self.wl
        out = []
        for l in range(sh.n_layers):
            desc = dbd.model_desc(replace(sh, n_layers=l + 1), act_pairs=wl.act_pairs)
            if self.wl.ctx_source == "hidden":
                h = self._hidden_rows(self.ctx, self.ctx + self.new)
                counts, hid = self.new, (h if h.numel() else None)
            else:
                counts, hid = np.zeros(wl.batch, np.int64), None
            _, tot = self._offsets(counts)
            self.call(self.ctx, counts, hid, logits=False, desc=desc)
            off = dbd.draft_residual_offset(desc, wl.batch, wl.block_len, wl.n_anchor, tot,
                                            wl.n_drafts, wl.temperature, self.cap)
            n = wl.batch * wl.block_len * sh.hidden
            torch.cuda.synchronize()
            x = self.last_ws[off:off + 4 * n].view(torch.float32)
            out.append(x.reshape(wl.batch, wl.block_len, sh.hidden).cpu().numpy())
        return out

    # ------------------------------------------------------------------ the oracle's view
    def cpu_weights(self):
        return {k: v.detach().to("cpu") for k, v in self.W.items()}

    def oracle_weights(self):
        """The weights as numpy arrays for the oracle, converted once: fp64 when that takes at
        most 20 GB of host memory, else fp32 (both exact for bf16 and fp32 values; the oracle
        upcasts fp32 to fp64 where it uses them)."""
        if self._oracle_w is None:
            n = sum(v.numel() for v in self.W.values())
            dt = torch.float64 if n * 8 <= 20e9 else torch.float32
            self._oracle_w = {k: v.detach().to(dt).cpu().numpy() for k, v in self.W.items()}
        return self._oracle_w

    def oracle_inputs(self, i):
        """(block tokens, hidden [C+n, L_t, H] or None, ctx_kv or None) of sequence i on CPU."""
        toks = self.tokens[i].to("cpu").numpy()
        if self.wl.ctx_source == "hidden":
            return toks, self.hidden[i].to("cpu"), None
        K, V = self.cache_kv
        C = int(self.ctx[i])
        kv = [(K[l, i, :, :C, :].to("cpu"), V[l, i, :, :C, :].to("cpu"))
              for l in range(self.shape.n_layers)]
        return toks, None, kv

    def gpu_cache(self, i, l, n_pos):
        """GPU cache contents of sequence i, layer l, positions < n_pos as (K, V) [kvh, n, hd]."""
        k = self.kv_k[l, i, :, :n_pos, :].float().cpu().numpy()
        v = dbd.unpack_values(self.kv_v[l, i]).float().cpu().numpy()[:, :n_pos, :]
        return k, v


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))
