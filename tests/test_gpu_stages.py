"""GPU parity of single stages: the projection GEMM (bf16 MFMA and fp32 paths) and the ingest
mix + RMSNorm, against the oracle's fp64 definitions on the same inputs."""
import numpy as np
import pytest
import torch

import block_diffusion_drafter_draft_amd as dbd
import synth
from oracle import drafter as od
from drafter_case import rel_l2

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("M,N,K", [(1, 1, 64), (128, 128, 64), (200, 300, 192), (512, 640, 4096),
                                   (480, 1000, 2560), (17, 2048, 1024), (235, 1024, 4096)])
def test_gemm_nt(dtype, M, N, K):
    print(f"gemm {dtype} M={M} N={N} K={K}", flush=True)
    g = torch.Generator(device=DEV).manual_seed(M * 7 + N * 3 + K)
    A = torch.randn((M, K), generator=g, device=DEV).to(dtype)
    B = (torch.randn((N, K), generator=g, device=DEV) * 0.02).to(dtype)
    C = torch.full((M, N), float("nan"), device=DEV)
    dbd.gemm_nt(A, B, C)
    torch.cuda.synchronize()
    ref = od.f64(A) @ od.f64(B).T
    # products of bf16 inputs are exact in fp32; only the fp32 accumulation rounds
    assert rel_l2(C.cpu().numpy(), ref) < 1e-5


@pytest.mark.parametrize("cfg", list(range(19)))
@pytest.mark.parametrize("M,N,K", [(200, 300, 192), (512, 640, 4096), (235, 1000, 2560),
                                   (16, 384, 4096)])
def test_gemm_nt_tile_configs(cfg, M, N, K):
    """Every bf16 tile configuration, with a workspace so the deep-ring tiles split K where
    their plan does; two calls in a row must agree bit for bit (the split partials are summed in
    split order)."""
    print(f"gemm cfg={cfg} M={M} N={N} K={K}", flush=True)
    g = torch.Generator(device=DEV).manual_seed(cfg * 131 + M + N + K)
    A = torch.randn((M, K), generator=g, device=DEV).to(torch.bfloat16)
    B = (torch.randn((N, K), generator=g, device=DEV) * 0.02).to(torch.bfloat16)
    wb = dbd.gemm_workspace_bytes(dbd.DBD_BF16, M, N, K, cfg)
    ws = torch.empty(max(wb, 1), dtype=torch.uint8, device=DEV) if wb else None
    C1 = torch.full((M, N), float("nan"), device=DEV)
    C2 = torch.full((M, N), float("nan"), device=DEV)
    dbd.gemm_nt(A, B, C1, tile_cfg=cfg, workspace=ws)
    dbd.gemm_nt(A, B, C2, tile_cfg=cfg, workspace=ws)
    torch.cuda.synchronize()
    ref = od.f64(A) @ od.f64(B).T
    assert rel_l2(C1.cpu().numpy(), ref) < 1e-5
    assert torch.equal(C1, C2)


@pytest.mark.parametrize("cfg", list(range(8, 19)))
@pytest.mark.parametrize("split", [2, 3, 5, 16])
@pytest.mark.parametrize("M,N,K", [(235, 1000, 2560), (512, 640, 4096)])
def test_gemm_nt_requested_split(cfg, split, M, N, K):
    """A requested split-K (partials added by the second kernel) over ragged M, N and k ranges
    that do not divide evenly; two calls in a row agree bit for bit."""
    print(f"gemm cfg={cfg} split={split} M={M} N={N} K={K}", flush=True)
    g = torch.Generator(device=DEV).manual_seed(cfg * 37 + split * 5 + M + K)
    A = torch.randn((M, K), generator=g, device=DEV).to(torch.bfloat16)
    B = (torch.randn((N, K), generator=g, device=DEV) * 0.02).to(torch.bfloat16)
    wb = dbd.gemm_workspace_bytes(dbd.DBD_BF16, M, N, K, cfg, split)
    assert wb > 0
    ws = torch.empty(wb, dtype=torch.uint8, device=DEV)
    C1 = torch.full((M, N), float("nan"), device=DEV)
    C2 = torch.full((M, N), float("nan"), device=DEV)
    dbd.gemm_nt(A, B, C1, tile_cfg=cfg, workspace=ws, split=split)
    dbd.gemm_nt(A, B, C2, tile_cfg=cfg, workspace=ws, split=split)
    torch.cuda.synchronize()
    ref = od.f64(A) @ od.f64(B).T
    assert rel_l2(C1.cpu().numpy(), ref) < 1e-5
    assert torch.equal(C1, C2)


@pytest.mark.parametrize("T", [77, 215])
@pytest.mark.parametrize("name", ["tiny-fp32", "qwen3-8b", "gpt-oss-20b"])
def test_mix_rmsnorm(name, T):
    """77 tokens: one workgroup per token and draft layer; 215 (the Qwen3-8B step's ingest):
    one workgroup per token for all its draft layers."""
    sh = synth.workload(name).shape
    W = synth.make_weights(sh, 0, DEV)
    hid = synth.make_hidden(sh, T, 0, 0, DEV)
    out = torch.empty((sh.n_layers, T, sh.hidden), dtype=hid.dtype, device=DEV)
    dbd.mix_rmsnorm(dbd.model_desc(sh), W["mix_logits"], W["mix_norm_w"], hid, out)
    torch.cuda.synchronize()
    Wc = {k: W[k].cpu() for k in ("mix_logits", "mix_norm_w")}
    tol = 1e-5 if sh.dtype == "f32" else 5e-3       # bf16 output rounding: 2^-9 relative
    for l in range(sh.n_layers):
        ref = od.context_features(sh, Wc, l, hid.cpu())
        assert rel_l2(out[l].float().cpu().numpy(), ref) < tol


def test_mix_rmsnorm_one_hot_selects_a_layer():
    sh = synth.workload("qwen3-8b").shape
    W = synth.make_weights(sh, 0, DEV)
    lg = torch.zeros_like(W["mix_logits"])
    lg[:, 4] = 1e4
    hid = synth.make_hidden(sh, 9, 0, 0, DEV)
    out = torch.empty((sh.n_layers, 9, sh.hidden), dtype=hid.dtype, device=DEV)
    dbd.mix_rmsnorm(dbd.model_desc(sh), lg, W["mix_norm_w"], hid, out)
    torch.cuda.synchronize()
    for l in range(sh.n_layers):
        ref = od.rmsnorm(od.f64(hid[:, 4, :]), od.f64(W["mix_norm_w"][l]), sh.rms_eps)
        assert rel_l2(out[l].float().cpu().numpy(), ref) < 5e-3


def test_mix_rmsnorm_strided_layer_major_input():
    """Target hidden states stored layer-major [L_t, T, H] are read through the strides."""
    sh = synth.workload("tiny-fp32").shape
    W = synth.make_weights(sh, 0, DEV)
    hid = synth.make_hidden(sh, 20, 0, 0, DEV)
    lm = hid.permute(1, 0, 2).contiguous()          # [L_t, T, H]
    view = lm.permute(1, 0, 2)                      # strides (H, T*H, 1)
    out = torch.empty((sh.n_layers, 20, sh.hidden), device=DEV)
    dbd.mix_rmsnorm(dbd.model_desc(sh), W["mix_logits"], W["mix_norm_w"], view, out)
    torch.cuda.synchronize()
    ref = od.context_features(sh, {k: W[k].cpu() for k in ("mix_logits", "mix_norm_w")}, 1,
                              hid.cpu())
    assert rel_l2(out[1].cpu().numpy(), ref) < 1e-5


@pytest.mark.parametrize("dtype,hidden", [("bf16", 6144), ("bf16", 8192), ("f32", 4096)])
def test_mix_rmsnorm_wide_rows(dtype, hidden):
    """Rows past 512 sixteen-byte chunks (the widest rows each dtype allows): two chunks per
    thread, the target layers loaded one ahead of the mixing instead of all at once."""
    sh = synth.DrafterShape(hidden=hidden, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=1024,
                            n_layers=3, n_target_layers=5, vocab=512, dtype=dtype)
    W = synth.make_weights(sh, 5, DEV)
    T = 13
    hid = synth.make_hidden(sh, T, 5, 0, DEV)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = torch.empty((sh.n_layers, T, sh.hidden), dtype=dt, device=DEV)
    dbd.mix_rmsnorm(dbd.model_desc(sh), W["mix_logits"], W["mix_norm_w"], hid, out)
    torch.cuda.synchronize()
    Wc = {k: W[k].cpu() for k in ("mix_logits", "mix_norm_w")}
    tol = 5e-3 if dtype == "bf16" else 1e-5
    for l in range(sh.n_layers):
        ref = od.context_features(sh, Wc, l, hid.cpu())
        assert rel_l2(out[l].float().cpu().numpy(), ref) < tol


@pytest.mark.parametrize("dtype,n_layers", [("bf16", 8), ("f32", 8), ("bf16", 12)])
def test_mix_rmsnorm_sixteen_target_layers(dtype, n_layers):
    """The mixing kernel at its target-layer limit: 16 target layers mixed into 8 and 12 draft
    layers.  37 tokens take one workgroup per token and draft layer; 150 tokens (the 12-layer
    case) take one workgroup per token and group of eight draft layers, two groups (8 + 4)."""
    sh = synth.DrafterShape(hidden=1024, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=2048,
                            n_layers=n_layers, n_target_layers=16, vocab=512, dtype=dtype)
    W = synth.make_weights(sh, 3, DEV)
    T = 37 if n_layers == 8 else 150
    hid = synth.make_hidden(sh, T, 3, 0, DEV)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = torch.empty((sh.n_layers, T, sh.hidden), dtype=dt, device=DEV)
    dbd.mix_rmsnorm(dbd.model_desc(sh), W["mix_logits"], W["mix_norm_w"], hid, out)
    torch.cuda.synchronize()
    Wc = {k: W[k].cpu() for k in ("mix_logits", "mix_norm_w")}
    tol = 5e-3 if dtype == "bf16" else 1e-5
    for l in range(sh.n_layers):
        ref = od.context_features(sh, Wc, l, hid.cpu())
        assert rel_l2(out[l].float().cpu().numpy(), ref) < tol
