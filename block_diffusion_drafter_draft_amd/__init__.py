"""Python binding of libdbd.so: block-diffusion drafting hot path on AMD MI355X (gfx950).

Argument marshalling only.  Every step of the path runs in the library's HIP kernels; torch
tensors provide device memory and the current HIP stream.  The library must be built
(``python -m block_diffusion_drafter_draft_amd.build``); importing without it raises.

Entry points (same names as the C ABI in include/dbd.h):
  draft_block, verify_greedy, select_streak
  draft_workspace_bytes, verify_workspace_bytes, select_workspace_bytes
  refine_block, refine_workspace_bytes (Mask-Predict update between draft_block passes)
Stage hooks used by the parity tests: sample_from_logits, mix_rmsnorm, gemm_nt,
draft_residual_offset.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdbd.so")

DBD_F32, DBD_BF16 = 0, 1
SEQ_NONFINITE, SEQ_BAD_LENGTH = 1, 2
ERRORS = {0: "OK", -1: "ARG", -2: "SHAPE", -3: "CAPACITY", -4: "WORKSPACE", -5: "UNSUPPORTED",
          -6: "HIP"}

_c = ctypes
_vp, _i32, _i64, _f32, _u64, _sz = (_c.c_void_p, _c.c_int32, _c.c_int64, _c.c_float,
                                    _c.c_uint64, _c.c_size_t)


class ModelDesc(_c.Structure):
    _fields_ = [("hidden", _i32), ("n_q_heads", _i32), ("n_kv_heads", _i32), ("head_dim", _i32),
                ("ffn", _i32), ("n_layers", _i32), ("n_target_layers", _i32), ("vocab", _i32),
                ("mask_token_id", _i32), ("dtype", _i32), ("rms_eps", _f32),
                ("act_pairs", _i32), ("rope_theta", _c.c_double), ("ctx_fusion", _i32),
                ("mix_raw", _i32), ("ctx_shared_kv", _i32)]


WEIGHT_FIELDS = ["mix_logits", "mix_norm_w", "wk_ctx", "wv_ctx", "attn_norm_w", "wq", "wk_draft",
                 "wv_draft", "wo", "mlp_norm_w", "w_gate", "w_up", "w_down", "final_norm_w",
                 "embed", "lm_head", "fc_w", "fc_norm_w"]


class Weights(_c.Structure):
    _fields_ = [(n, _vp) for n in WEIGHT_FIELDS]


class DbdError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"dbd error {code} ({ERRORS.get(code, '?')}): {msg}")
        self.code = code


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m block_diffusion_drafter_draft_amd.build`")
        L = _c.CDLL(LIB_PATH)
        sig = {
            "dbd_last_error": (_c.c_char_p, []),
            "dbd_draft_workspace_bytes": (_i32, [_c.POINTER(ModelDesc), _i32, _i32, _i32, _i32,
                                                 _i32, _f32, _i32, _c.POINTER(_sz)]),
            "draft_block": (_i32, [_c.POINTER(ModelDesc), _c.POINTER(Weights), _i32, _i32, _i32,
                                   _vp, _vp, _i64, _i64, _i32, _vp, _vp, _vp, _vp, _i32, _i32,
                                   _f32, _u64, _vp, _vp, _vp, _vp, _sz, _vp]),
            "dbd_verify_workspace_bytes": (_i32, [_i32, _i32, _i32, _c.POINTER(_sz)]),
            "verify_greedy": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp,
                                     _vp, _sz, _vp]),
            "verify_greedy_noalloc": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp,
                                             _vp, _vp, _vp]),
            "dbd_verify_sample_workspace_bytes": (_i32, [_i32, _i32, _i32, _i32,
                                                         _c.POINTER(_sz)]),
            "verify_sample": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _f32, _f32,
                                     _u64, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
            "dbd_select_workspace_bytes": (_i32, [_i32, _i32, _i32, _i32, _c.POINTER(_sz)]),
            "select_streak": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp,
                                     _vp, _vp, _vp, _sz, _vp]),
            "dbd_sample_workspace_bytes": (_i32, [_i32, _i32, _i32, _c.POINTER(_sz)]),
            "dbd_sample_top_p_workspace_bytes": (_i32, [_i32, _i32, _i32, _c.POINTER(_sz)]),
            "dbd_refine_workspace_bytes": (_i32, [_i32, _i32, _i32, _c.POINTER(_sz)]),
            "refine_block": (_i32, [_vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _sz,
                                    _vp]),
            "dbd_sample_top_p": (_i32, [_vp, _i32, _i32, _i32, _i32, _f32, _f32, _u64, _vp,
                                        _vp, _sz, _vp]),
            "dbd_sample_from_logits": (_i32, [_vp, _i32, _i32, _i32, _i32, _f32, _u64, _vp, _vp,
                                              _sz, _vp]),
            "dbd_mix_rmsnorm": (_i32, [_c.POINTER(ModelDesc), _vp, _vp, _vp, _i64, _i64, _i32,
                                       _vp, _vp]),
            "dbd_draft_residual_offset": (_i32, [_c.POINTER(ModelDesc), _i32, _i32, _i32, _i32,
                                                 _i32, _f32, _i32, _c.POINTER(_sz)]),
            "dbd_gemm_workspace_bytes": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32,
                                                _c.POINTER(_sz)]),
            "dbd_gemm_nt": (_i32, [_i32, _vp, _vp, _vp, _i32, _i32, _i32, _i64, _i64, _i64, _i32,
                                   _i32, _vp, _sz, _vp]),
            "dbd_gemm_override": (_i32, [_i32, _i32, _i32]),
            "dbd_attn_override": (_i32, [_i32, _i32]),
            "dbd_timing_enable": (_i32, [_i32]),
            "dbd_timing_reset": (_i32, []),
            "dbd_timing_read": (_i32, [_i32, _c.POINTER(_c.c_double), _c.POINTER(_i64)]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(rc):
    if rc != 0:
        raise DbdError(rc, lib().dbd_last_error().decode())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream, *tensors):
    if stream is not None:
        return stream
    import torch
    for t in tensors:
        if t is not None and t.is_cuda:
            return torch.cuda.current_stream(t.device).cuda_stream
    return None


def model_desc(shape, dtype=None, act_pairs=0) -> ModelDesc:
    """ModelDesc from an object with the drafter's shape attributes (e.g. synth.DrafterShape);
    act_pairs=1 feeds the projection GEMMs bf16 (high, low) activation pairs."""
    dt = dtype if dtype is not None else shape.dtype
    code = {"f32": DBD_F32, "bf16": DBD_BF16, DBD_F32: DBD_F32, DBD_BF16: DBD_BF16}[dt]
    return ModelDesc(shape.hidden, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.ffn,
                     shape.n_layers, shape.n_target_layers, shape.vocab,
                     shape.vocab - 1 if not hasattr(shape, "mask_token_id")
                     else shape.mask_token_id, code, float(shape.rms_eps), int(act_pairs),
                     float(shape.rope_theta),
                     1 if getattr(shape, "ctx_fusion", "mix") == "fc" else 0,
                     int(bool(getattr(shape, "mix_raw", False))),
                     int(bool(getattr(shape, "ctx_shared_kv", False))))


def kv_cache_shapes(shape, batch, ctx_capacity):
    """Shapes of the K and V cache tensors (see the KV-cache layout in include/dbd.h)."""
    L, kvh, hd = shape.n_layers, shape.n_kv_heads, shape.head_dim
    return (L, batch, kvh, ctx_capacity, hd), (L, batch, kvh, ctx_capacity // 8, hd, 8)


def pack_values(v):
    """[..., P, hd] values by position (P a multiple of 8) -> the cache's [..., P/8, hd, 8]."""
    *lead, P, hd = v.shape
    return v.reshape(*lead, P // 8, 8, hd).transpose(-1, -2)


def unpack_values(vb):
    """Inverse of pack_values: [..., P/8, hd, 8] -> [..., P, hd]."""
    *lead, B8, hd, e = vb.shape
    return vb.transpose(-1, -2).reshape(*lead, B8 * e, hd)


def weights_struct(w: dict) -> Weights:
    """Weights from a dict of device tensors keyed by the field names (missing keys -> NULL)."""
    return Weights(*[_ptr(w.get(n)) for n in WEIGHT_FIELDS])


def draft_workspace_bytes(desc, batch, block_len, n_anchor, max_new_tokens, n_drafts,
                          temperature, ctx_capacity) -> int:
    out = _sz(0)
    _check(lib().dbd_draft_workspace_bytes(_c.byref(desc), batch, block_len, n_anchor,
                                           max_new_tokens, n_drafts, float(temperature),
                                           ctx_capacity, _c.byref(out)))
    return out.value


def draft_block(desc, weights, block_tokens, target_hidden_new, new_offsets, ctx_len, kv_k,
                kv_v, draft_tokens, workspace, n_new_total, n_drafts=1, temperature=0.0, seed=0,
                n_anchor=1, hid_token_stride=None, hid_layer_stride=None, logits_out=None,
                seq_status=None, stream=None):
    """Enqueue one drafter forward + drafting (see draft_block in include/dbd.h).

    block_tokens [N, B] int32; target_hidden_new [T, L_t, H] (or strided) or None;
    new_offsets [N+1] int32; ctx_len [N] int32; kv_k [L, N, kvh, cap, hd]; kv_v [L, N, kvh, hd,
    cap]; draft_tokens [N, K, D] int32 out; workspace uint8 tensor."""
    N, B = block_tokens.shape
    cap = kv_k.shape[3]
    ts = hid_token_stride if hid_token_stride is not None else (
        target_hidden_new.stride(0) if target_hidden_new is not None else 0)
    ls = hid_layer_stride if hid_layer_stride is not None else (
        target_hidden_new.stride(1) if target_hidden_new is not None else 0)
    _check(lib().draft_block(
        _c.byref(desc), _c.byref(weights), N, B, n_anchor, _ptr(block_tokens),
        _ptr(target_hidden_new), ts, ls, int(n_new_total), _ptr(new_offsets), _ptr(ctx_len),
        _ptr(kv_k), _ptr(kv_v), cap, n_drafts, float(temperature), int(seed) & (2**64 - 1),
        _ptr(draft_tokens), _ptr(logits_out), _ptr(seq_status), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream, block_tokens)))


def draft_residual_offset(desc, batch, block_len, n_anchor, n_new_total, n_drafts, temperature,
                          ctx_capacity) -> int:
    """Byte offset of the fp32 residual [batch * block_len, H] in the workspace of a draft_block
    call with these arguments (test hook for per-layer parity)."""
    out = _sz(0)
    _check(lib().dbd_draft_residual_offset(_c.byref(desc), batch, block_len, n_anchor,
                                           int(n_new_total), n_drafts, float(temperature),
                                           ctx_capacity, _c.byref(out)))
    return out.value


def verify_workspace_bytes(batch, n_rows, vocab) -> int:
    out = _sz(0)
    _check(lib().dbd_verify_workspace_bytes(batch, n_rows, vocab, _c.byref(out)))
    return out.value


def verify_greedy(target_logits, draft_tokens, n_accepted, bonus, committed, workspace,
                  row_flags=None, stream=None):
    """target_logits [N, R, V] fp32; draft_tokens [N, D] int32 (row stride taken from the
    tensor)."""
    N, R, V = target_logits.shape
    D = draft_tokens.shape[-1]
    _check(lib().verify_greedy(
        _ptr(target_logits), _ptr(draft_tokens), draft_tokens.stride(0), N, D, R, V,
        _ptr(n_accepted), _ptr(bonus), _ptr(committed), _ptr(row_flags), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream, target_logits)))


STATIC_SCRATCH_BYTES = 4 << 20      # DBD_STATIC_SCRATCH_BYTES


def verify_greedy_noalloc(target_logits, draft_tokens, n_accepted, bonus, committed,
                          row_flags=None, stream=None):
    """verify_greedy without a workspace: the library's static device scratch holds the
    partials (calls that overlap on one GPU race)."""
    N, R, V = target_logits.shape
    D = draft_tokens.shape[-1]
    _check(lib().verify_greedy_noalloc(
        _ptr(target_logits), _ptr(draft_tokens), draft_tokens.stride(0), N, D, R, V,
        _ptr(n_accepted), _ptr(bonus), _ptr(committed), _ptr(row_flags),
        _stream(stream, target_logits)))


def verify_sample_workspace_bytes(batch, n_draft, n_rows, vocab) -> int:
    out = _sz(0)
    _check(lib().dbd_verify_sample_workspace_bytes(batch, n_draft, n_rows, vocab, _c.byref(out)))
    return out.value


def verify_sample(target_logits, draft_logits, draft_tokens, t_target, t_draft, seed,
                  n_accepted, bonus, committed, workspace, row_flags=None, stream=None):
    """target_logits [N, R, V] fp32; draft_logits [N, D, V] fp32; draft_tokens [N, D] int32 (row
    stride taken from the tensor)."""
    N, R, V = target_logits.shape
    D = draft_tokens.shape[-1]
    _check(lib().verify_sample(
        _ptr(target_logits), _ptr(draft_logits), _ptr(draft_tokens), draft_tokens.stride(0), N,
        D, R, V, float(t_target), float(t_draft), int(seed) & ((1 << 64) - 1), _ptr(n_accepted),
        _ptr(bonus), _ptr(committed), _ptr(row_flags), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream, target_logits)))


def select_workspace_bytes(batch, n_drafts, n_rows, vocab) -> int:
    out = _sz(0)
    _check(lib().dbd_select_workspace_bytes(batch, n_drafts, n_rows, vocab, _c.byref(out)))
    return out.value


def select_streak(verifier_logits, drafts, selected, n_accepted, bonus, committed, workspace,
                  scores=None, row_flags=None, stream=None):
    """verifier_logits [N, K, R, V] fp32; drafts [N, K, G] int32."""
    N, K, R, V = verifier_logits.shape
    G = drafts.shape[2]
    _check(lib().select_streak(
        _ptr(verifier_logits), _ptr(drafts), N, K, G, R, V, _ptr(selected), _ptr(scores),
        _ptr(n_accepted), _ptr(bonus), _ptr(committed), _ptr(row_flags), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream, verifier_logits)))


def sample_workspace_bytes(batch, n_draft, vocab) -> int:
    out = _sz(0)
    _check(lib().dbd_sample_workspace_bytes(batch, n_draft, vocab, _c.byref(out)))
    return out.value


def sample_from_logits(logits, n_drafts, temperature, seed, out, workspace, stream=None):
    """logits [N, D, V] fp32 -> out [N, K, D] int32 (the drafting stage of draft_block)."""
    N, D, V = logits.shape
    _check(lib().dbd_sample_from_logits(
        _ptr(logits), N, D, V, n_drafts, float(temperature), int(seed) & (2**64 - 1), _ptr(out),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream, logits)))


def sample_top_p_workspace_bytes(batch, n_draft, vocab) -> int:
    out = _sz(0)
    _check(lib().dbd_sample_top_p_workspace_bytes(batch, n_draft, vocab, _c.byref(out)))
    return out.value


def sample_top_p(logits, n_drafts, temperature, top_p, seed, out, workspace, stream=None):
    """logits [N, D, V] fp32 -> out [N, K, D] int32, each draw restricted to its top-p nucleus."""
    N, D, V = logits.shape
    _check(lib().dbd_sample_top_p(
        _ptr(logits), N, D, V, n_drafts, float(temperature), float(top_p),
        int(seed) & (2**64 - 1), _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream, logits)))


def refine_workspace_bytes(batch, n_draft, vocab) -> int:
    out = _sz(0)
    _check(lib().dbd_refine_workspace_bytes(batch, n_draft, vocab, _c.byref(out)))
    return out.value


def refine_block(logits, block_tokens, conf, n_anchor, mask_id, n_remask, workspace,
                 stream=None):
    """One refinement update: logits [N, D, V] fp32 of the forward that read block_tokens [N, B]
    int32; block_tokens and conf [N, D] uint64 (stored as int64) are updated in place."""
    N, D, V = logits.shape
    _check(lib().refine_block(
        _ptr(logits), N, block_tokens.shape[1], n_anchor, V, mask_id, n_remask,
        _ptr(block_tokens), _ptr(conf), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream, logits)))


def mix_rmsnorm(desc, mix_logits, mix_norm_w, hidden, out, stream=None):
    """hidden [T, L_t, H] (strided ok) -> out [L_d, T, H] (the ingest mixing stage)."""
    _check(lib().dbd_mix_rmsnorm(
        _c.byref(desc), _ptr(mix_logits), _ptr(mix_norm_w), _ptr(hidden), hidden.stride(0),
        hidden.stride(1), hidden.shape[0], _ptr(out), _stream(stream, hidden)))


def gemm_workspace_bytes(dtype, M, N, K, tile_cfg=-1, split=0):
    """Workspace bytes gemm_nt needs to split K for this shape, tile and split (0: it does not)."""
    out = _sz(0)
    _check(lib().dbd_gemm_workspace_bytes(dtype, M, N, K, int(tile_cfg), int(split),
                                          _c.byref(out)))
    return out.value


def gemm_nt(A, B, C, tile_cfg=-1, workspace=None, stream=None, split=0):
    """C[M, N] fp32 = A[M, K] . B[N, K]^T with A, B both fp32 or both bf16; tile_cfg picks the
    bf16 block tile (-1: the library's choice).  With a workspace (gemm_workspace_bytes) the
    deep-ring tiles may split K over several workgroups: split 0 lets the library choose, 1 does
    not split, S > 1 splits S ways (a second kernel adds the partials in split order)."""
    import torch
    dt = DBD_BF16 if A.dtype == torch.bfloat16 else DBD_F32
    M, K = A.shape
    N = B.shape[0]
    wb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().dbd_gemm_nt(dt, _ptr(A), _ptr(B), _ptr(C), M, N, K, A.stride(0), B.stride(0),
                             C.stride(0), int(tile_cfg), int(split), _ptr(workspace), wb,
                             _stream(stream, A)))


def gemm_override(stage, tile_cfg=-1, split=0):
    """Replace the tile / split-K choice of one draft_block GEMM stage (a name of STAGES starting
    with "gemm_"); -1 / 0 restore the library's choice.  Set before sizing the workspace."""
    _check(lib().dbd_gemm_override(STAGES.index(stage), int(tile_cfg), int(split)))


def attn_override(workgroups=0, depth=0):
    """Replace the bf16 attention kernel's workgroup count and chunks loaded ahead (0, 0: the
    library's choice).  Set before sizing the workspace."""
    _check(lib().dbd_attn_override(int(workgroups), int(depth)))


# Stage order of DBD_STAGE_* in include/dbd.h.
STAGES = ["prep", "mix", "gemm_ctxkv", "rownorm", "gemm_qkv", "attn", "gemm_o", "gemm_gateup",
          "gemm_down", "gemm_lmhead", "draft", "verify", "select"]


def timing_enable(on: bool = True):
    """Bracket every library launch with HIP events on its stream (benchmarks only)."""
    _check(lib().dbd_timing_enable(1 if on else 0))


def timing_reset():
    _check(lib().dbd_timing_reset())


def timing_read():
    """{stage: (kernel milliseconds, launches)} since the last reset (synchronises)."""
    out = {}
    for i, name in enumerate(STAGES):
        ms, n = _c.c_double(0.0), _i64(0)
        _check(lib().dbd_timing_read(i, _c.byref(ms), _c.byref(n)))
        out[name] = (ms.value, n.value)
    return out
