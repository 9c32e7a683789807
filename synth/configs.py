"""Drafter shapes and the five synthetic workloads.

Shapes follow what the pages state about the drafters (DFlare page, evaluation section: Qwen
drafters use 7 draft layers, block 16 and 9 target layers; GPT-OSS uses 8, 8 and 7.  SpecDiff-2
notes, experimental setup: a 7B diffusion drafter, one denoising step, a window of 32 masks) and
the published sizes of the named model families.  Everything else (batch, context lengths,
distributions) is the synthetic stand-in for the pages' benchmark suites, which are not used.
"""
from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class DrafterShape:
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    n_layers: int              # L_d, draft layers
    n_target_layers: int       # L_t, mixed target hidden layers (0: context K/V given in a cache)
    vocab: int
    dtype: str                 # "f32" or "bf16"
    rms_eps: float = 1e-6
    rope_theta: float = 1e6
    # context-feature path: "mix" = per-draft-layer mixing of the target layers then RMSNorm;
    # "fc" = one fully connected fusion of the concatenated target layers then RMSNorm, shared
    # by every draft layer
    ctx_fusion: str = "mix"
    mix_raw: bool = False          # mixing coefficients used as given (no softmax)
    ctx_shared_kv: bool = False    # context K/V projected with the draft block's K/V weights

    @property
    def mask_token_id(self) -> int:
        return self.vocab - 1

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim


@dataclass(frozen=True)
class Workload:
    name: str
    shape: DrafterShape
    batch: int
    block_len: int             # forward width B, anchor counted
    n_anchor: int              # 1: [anchor, MASK...]; 0: all masks
    n_drafts: int              # K joint drafts per block
    temperature: float         # <= 0: argmax drafts
    ctx_lo: int                # cached context length range (inclusive)
    ctx_hi: int
    ctx_source: str            # "hidden": cache filled from target hidden states; "cache": given K/V
    verify: str                # "greedy" or "streak"
    verify_rows: int           # rows of target/verifier logits per draft
    planted_alpha: float       # per-position success probability used to plant acceptance
    logit_std: float = 2.0
    fixed_new: int = -1        # >= 0: every sequence ingests exactly this many new positions
    act_pairs: int = 0         # 1: the library feeds its GEMMs bf16 (high, low) activation pairs
    seed: int = 0
    notes: str = ""

    @property
    def n_draft(self) -> int:
        """D, drafted positions per block."""
        return self.block_len - self.n_anchor

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


TINY = DrafterShape(hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=688, n_layers=2,
                    n_target_layers=3, vocab=1024, dtype="f32")
QWEN3_4B = DrafterShape(hidden=2560, n_q_heads=32, n_kv_heads=8, head_dim=128, ffn=9728,
                        n_layers=7, n_target_layers=9, vocab=151936, dtype="bf16")
QWEN3_8B = DrafterShape(hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, ffn=12288,
                        n_layers=7, n_target_layers=9, vocab=151936, dtype="bf16")
GPT_OSS_20B = DrafterShape(hidden=2880, n_q_heads=64, n_kv_heads=8, head_dim=64, ffn=11520,
                           n_layers=8, n_target_layers=7, vocab=201088, dtype="bf16")
# DFlash-style context path (fully connected fusion, one K/V projection for context and block)
# and the mixing ablations, on the tiny and Qwen3-8B shapes
TINY_FC = replace(TINY, ctx_fusion="fc", ctx_shared_kv=True)
TINY_ABL = replace(TINY, mix_raw=True, ctx_shared_kv=True)
QWEN3_8B_FC = replace(QWEN3_8B, ctx_fusion="fc", ctx_shared_kv=True)
SPECDIFF2_7B = DrafterShape(hidden=3584, n_q_heads=28, n_kv_heads=4, head_dim=128, ffn=18944,
                            n_layers=28, n_target_layers=0, vocab=152064, dtype="bf16")

# Planted per-position success rates: alpha with sum_{m<=D} alpha^m + 1 equal to the acceptance
# lengths the pages report (DFlare page, results at temperature 0: 7.47 / 7.33 / 4.93; SpecDiff-2
# notes, section 7.1: average streak 5.98).
WORKLOADS = {
    "tiny-fp32": Workload(
        name="tiny-fp32", shape=TINY, batch=1, block_len=8, n_anchor=1, n_drafts=1,
        temperature=0.0, ctx_lo=56, ctx_hi=56, ctx_source="hidden", verify="greedy",
        verify_rows=8, planted_alpha=0.7, fixed_new=8,
        notes="context 64 = 56 cached + 8 ingested; fp32 path"),
    "tiny-dflash-fp32": Workload(
        name="tiny-dflash-fp32", shape=TINY_FC, batch=1, block_len=8, n_anchor=1, n_drafts=1,
        temperature=0.0, ctx_lo=56, ctx_hi=56, ctx_source="hidden", verify="greedy",
        verify_rows=8, planted_alpha=0.7, fixed_new=8,
        notes="fully connected context fusion, shared K/V projection; fp32 path"),
    "tiny-ablate-fp32": Workload(
        name="tiny-ablate-fp32", shape=TINY_ABL, batch=1, block_len=8, n_anchor=1, n_drafts=1,
        temperature=0.0, ctx_lo=56, ctx_hi=56, ctx_source="hidden", verify="greedy",
        verify_rows=8, planted_alpha=0.7, fixed_new=8,
        notes="mixing without softmax, shared K/V projection; fp32 path"),
    "qwen3-8b-dflash": Workload(
        name="qwen3-8b-dflash", shape=QWEN3_8B_FC, batch=32, block_len=16, n_anchor=1,
        n_drafts=1, temperature=0.0, ctx_lo=256, ctx_hi=3072, ctx_source="hidden",
        verify="greedy", verify_rows=16, planted_alpha=0.8818,
        notes="the bench workload with the DFlash-style context path"),
    "qwen3-4b": Workload(
        name="qwen3-4b", shape=QWEN3_4B, batch=1, block_len=16, n_anchor=1, n_drafts=1,
        temperature=0.0, ctx_lo=1024, ctx_hi=1024, ctx_source="hidden", verify="greedy",
        verify_rows=16, planted_alpha=0.8851),
    "qwen3-8b": Workload(
        name="qwen3-8b", shape=QWEN3_8B, batch=32, block_len=16, n_anchor=1, n_drafts=1,
        temperature=0.0, ctx_lo=256, ctx_hi=3072, ctx_source="hidden", verify="greedy",
        verify_rows=16, planted_alpha=0.8818),
    "gpt-oss-20b": Workload(
        name="gpt-oss-20b", shape=GPT_OSS_20B, batch=16, block_len=8, n_anchor=1, n_drafts=1,
        temperature=1.0, ctx_lo=4096, ctx_hi=4096, ctx_source="hidden", verify="greedy",
        verify_rows=8, planted_alpha=0.8552),
    "specdiff2-7b": Workload(
        name="specdiff2-7b", shape=SPECDIFF2_7B, batch=4, block_len=32, n_anchor=0, n_drafts=8,
        temperature=1.5, ctx_lo=2048, ctx_hi=2048, ctx_source="cache", verify="streak",
        verify_rows=32, planted_alpha=0.8332, fixed_new=0, act_pairs=1,
        notes="28 layers: bf16 activation pairs keep the logits within 2e-2 of the fp64 "
              "oracle; at 128 rows the GEMMs are HBM-bound, so the pairs cost little"),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]
