"""The C-ABI library loads, exports every function include/dbd.h declares, and rejects bad
arguments on the host before any launch (no GPU needed: every call here returns before touching
the device)."""
import ctypes
import os
import re

import pytest

import block_diffusion_drafter_draft_amd as dbd
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


# These calls pass placeholder addresses that the host-side validation must reject before any
# launch.  They are host-logic tests: where a GPU is visible they are not run at all, so that a
# validation bug can never turn into a launch with a placeholder address.
pytestmark = pytest.mark.skipif(_gpu_visible(), reason="host-logic test; runs where no GPU is "
                                "visible")
HEADER = os.path.join(ROOT, "include", "dbd.h")


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while", "sizeof")))


def test_header_declares_the_three_entry_points():
    fns = header_functions()
    for f in ("draft_block", "verify_greedy", "select_streak"):
        assert f in fns


def test_library_exports_every_declared_function():
    L = dbd.lib()
    missing = [f for f in header_functions() if not hasattr(L, f)]
    assert not missing, missing


def test_struct_layouts_match_header(tmp_path):
    """Every field offset and the size of dbd_model_desc and dbd_weights, as the C compiler lays
    them out from include/dbd.h, equal the ctypes mirrors of the binding."""
    import shutil
    import subprocess
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = src[: src.index("} dbd_weights;")]
    body = body[body.rindex("typedef struct {"):]
    names = re.findall(r"\*\s*(\w+);", body)
    assert names == dbd.WEIGHT_FIELDS
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    probe = tmp_path / "probe.c"
    lines = ['#include <stddef.h>', '#include <stdio.h>', f'#include "{HEADER}"', "int main(void) {"]
    for st, cls in (("dbd_model_desc", dbd.ModelDesc), ("dbd_weights", dbd.Weights)):
        lines.append(f'  printf("{st} size %zu\\n", sizeof({st}));')
        for f, _ in cls._fields_:
            lines.append(f'  printf("{st} {f} %zu\\n", offsetof({st}, {f}));')
    lines.append("  return 0;\n}")
    probe.write_text("\n".join(lines))
    exe = tmp_path / "probe"
    subprocess.run([cc, str(probe), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    got = {tuple(l.split()[:2]): int(l.split()[2]) for l in out if l.strip()}
    for st, cls in (("dbd_model_desc", dbd.ModelDesc), ("dbd_weights", dbd.Weights)):
        assert got[(st, "size")] == ctypes.sizeof(cls), st
        for f, _ in cls._fields_:
            assert got[(st, f)] == getattr(cls, f).offset, (st, f)


def _desc(name="qwen3-8b", **kw):
    d = dbd.model_desc(synth.workload(name).shape)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def _ws(desc, **kw):
    args = dict(batch=32, block_len=16, n_anchor=1, max_new_tokens=256, n_drafts=1,
                temperature=0.0, ctx_capacity=3136)
    args.update(kw)
    return dbd.draft_workspace_bytes(desc, **args)


def test_workspace_query_is_positive_and_monotone():
    d = _desc()
    a = _ws(d)
    b = _ws(d, batch=64)
    c = _ws(d, temperature=1.0)
    assert 0 < a < b and a < c
    assert a % 256 == 0


@pytest.mark.parametrize("name,cap,new", [("qwen3-8b", 3136, 256), ("qwen3-8b", 1024, 64),
                                          ("specdiff2-7b", 320, 0), ("tiny-fp32", 448, 40)])
def test_workspace_for_a_batch_covers_every_smaller_batch(name, cap, new):
    """The query sizes a workspace for at most `max_batch` sequences: the split-K tiles and
    splits and the attention split change with the number of rows, so a smaller batch can need
    more split partials (3 or 4 sequences of 16 rows take the skinny split-K tiles); the query
    for a batch must still cover every smaller one."""
    d = _desc(name)
    sizes = [_ws(d, batch=b, ctx_capacity=cap, block_len=16, n_anchor=1, max_new_tokens=new)
             for b in range(1, 41)]
    assert all(x <= y for x, y in zip(sizes, sizes[1:])), sizes


def test_workspace_for_an_ingest_covers_every_smaller_one():
    """Likewise for at most `max_new_tokens` ingested rows (the context K/V projection takes
    split-K tiles at a few dozen rows)."""
    d = _desc("qwen3-8b")
    sizes = [_ws(d, batch=2, max_new_tokens=t) for t in range(1, 300)]
    assert all(x <= y for x, y in zip(sizes, sizes[1:]))


@pytest.mark.parametrize("field,value,code", [
    ("head_dim", 96, -2),            # only 64 / 128
    ("n_kv_heads", 5, -2),           # 32 % 5 != 0
    ("dtype", 7, -1),
    ("vocab", 1 << 18, -2),
    ("hidden", 4100, -2),            # bf16 needs multiples of 64
    ("n_target_layers", 17, -5),
])
def test_bad_model_desc_rejected(field, value, code):
    with pytest.raises(dbd.DbdError) as e:
        _ws(_desc(**{field: value}))
    assert e.value.code == code


@pytest.mark.parametrize("kw,code", [
    (dict(block_len=65), -2),
    (dict(n_anchor=2), -1),
    (dict(n_drafts=2, temperature=0.0), -1),     # argmax drafting with K > 1
    (dict(ctx_capacity=1000), -3),              # not a multiple of 64
    (dict(ctx_capacity=8), -3),                 # smaller than the block
    (dict(batch=0), -1),
])
def test_bad_draft_shape_rejected(kw, code):
    with pytest.raises(dbd.DbdError) as e:
        _ws(_desc(), **kw)
    assert e.value.code == code


def test_draft_block_null_pointers_rejected_before_launch():
    L = dbd.lib()
    d = _desc()
    w = dbd.Weights()
    rc = L.draft_block(ctypes.byref(d), ctypes.byref(w), 32, 16, 1, None, None, 0, 0, 0, None,
                       None, None, None, 3136, 1, 0.0, 0, None, None, None, None, 0, None)
    assert rc == -1 and b"NULL" in L.dbd_last_error()


def test_draft_block_small_workspace_rejected():
    L = dbd.lib()
    d = _desc()
    fake = 1 << 20                                  # never dereferenced: rejected on the host
    w = dbd.Weights(*([fake] * 16))
    rc = L.draft_block(ctypes.byref(d), ctypes.byref(w), 32, 16, 1, fake, fake, 8 * 9 * 4096,
                       4096, 100, fake, fake, fake, fake, 3136, 1, 0.0, 0, fake, None, None,
                       fake, 1024, None)
    assert rc == -4 and b"workspace" in L.dbd_last_error()


def test_draft_block_misaligned_hidden_rejected():
    L = dbd.lib()
    d = _desc()
    fake = 1 << 20
    w = dbd.Weights(*([fake] * 16))
    rc = L.draft_block(ctypes.byref(d), ctypes.byref(w), 32, 16, 1, fake, fake + 2,
                       8 * 9 * 4096, 4096, 100, fake, fake, fake, fake, 3136, 1, 0.0, 0, fake,
                       None, None, fake, 1 << 40, None)
    assert rc == -2


def test_drafter_without_mixing_rejects_ingest():
    d = dbd.model_desc(synth.workload("specdiff2-7b").shape)
    with pytest.raises(dbd.DbdError) as e:
        dbd.draft_workspace_bytes(d, 4, 32, 0, 10, 8, 1.5, 2112)
    assert e.value.code == -1


@pytest.mark.parametrize("args,code", [
    ((2, 3, 1, 4, 100), -2),       # n_rows not in {D, D+1}
    ((2, 65, 65, 66, 100), -5),    # D > 64
    ((2, 3, 3, 3, 1 << 18), -1),   # vocab too large
    ((2, 3, 2, 4, 100), -2),       # draft_stride < D
])
def test_verify_validation(args, code):
    L = dbd.lib()
    fake = 1 << 20
    batch, D, stride, R, V = args
    rc = L.verify_greedy(fake, fake, stride, batch, D, R, V, fake, fake, fake, None, fake,
                         1 << 30, None)
    assert rc == code


def test_verify_noalloc_validation():
    """verify_greedy_noalloc validates like verify_greedy and rejects, before any HIP call, a call
    whose partials exceed the static scratch (the size is checked here against the workspace
    query first, so the rejected case really is over the limit)."""
    L = dbd.lib()
    fake = 1 << 20
    N, D, R, V = 128, 64, 65, (1 << 18) - 1
    assert dbd.verify_workspace_bytes(N, R, V) > dbd.STATIC_SCRATCH_BYTES
    rc = L.verify_greedy_noalloc(fake, fake, D, N, D, R, V, fake, fake, fake, None, None)
    assert rc == -4 and b"static limit" in L.dbd_last_error()
    assert L.verify_greedy_noalloc(fake, fake, 3, 2, 3, 5, 100, fake, fake, fake, None,
                                   None) == -2
    assert L.verify_greedy_noalloc(None, fake, 3, 2, 3, 3, 100, fake, fake, fake, None,
                                   None) == -1
    assert L.verify_greedy_noalloc(fake, fake, 65, 2, 65, 66, 100, fake, fake, fake, None,
                                   None) == -5


def test_select_validation():
    L = dbd.lib()
    fake = 1 << 20
    rc = L.select_streak(fake, fake, 2, 8, 32, 34, 1000, fake, None, fake, fake, fake, None, fake,
                         1 << 30, None)
    assert rc == -2
    rc = L.select_streak(fake, fake, 2, 8, 32, 32, 1000, fake, None, fake, fake, fake, None, fake,
                         16, None)
    assert rc == -4
    rc = L.select_streak(fake, fake, 2, 65, 32, 32, 1000, fake, None, fake, fake, fake, None, fake,
                         1 << 30, None)
    assert rc == -5


def test_sample_validation():
    L = dbd.lib()
    fake = 1 << 20
    assert L.dbd_sample_from_logits(fake, 2, 3, 100, 2, 0.0, 0, fake, fake, 1 << 30, None) == -1
    assert L.dbd_sample_from_logits(fake, 2, 3, 100, 1, 1.0, 0, fake, fake, 8, None) == -4


def test_gemm_validation():
    L = dbd.lib()
    fake = 1 << 20
    assert L.dbd_gemm_nt(1, fake, fake, fake, 4, 4, 48, 48, 48, 4, -1, 0, None, 0, None) == -2
    assert L.dbd_gemm_nt(0, fake, fake, fake, 4, 4, 8, 4, 8, 4, -1, 0, None, 0, None) == -2
    assert L.dbd_gemm_nt(3, fake, fake, fake, 4, 4, 8, 8, 8, 4, -1, 0, None, 0, None) == -1
    assert L.dbd_gemm_nt(1, fake, fake, fake, 4, 4, 64, 64, 64, 4, 19, 0, None, 0, None) == -1
    for bad in (17, -1):
        assert L.dbd_gemm_nt(1, fake, fake, fake, 4, 4, 64, 64, 64, 4, 8, bad, None, 0, None) == -1
        with pytest.raises(dbd.DbdError):
            dbd.gemm_workspace_bytes(dbd.DBD_BF16, 4, 4, 64, 8, bad)
    # a split-K shape with a workspace that is too small, or misaligned
    need = dbd.gemm_workspace_bytes(dbd.DBD_BF16, 512, 4096, 4096, 8)
    assert need > 0
    assert L.dbd_gemm_nt(1, fake, fake, fake, 512, 4096, 4096, 4096, 4096, 4096, 8, 0, fake,
                         need - 1, None) == -4
    assert L.dbd_gemm_nt(1, fake, fake, fake, 512, 4096, 4096, 4096, 4096, 4096, 8, 0, fake + 16,
                         need, None) == -4
    assert dbd.gemm_workspace_bytes(dbd.DBD_F32, 512, 4096, 4096) == 0


def test_gemm_requested_split_sizes_workspace():
    """A requested split S sizes one fp32 tile per (output tile, split); no split and the
    pipelined tiles need nothing; a split is capped at K / 64."""
    M, N, K = 512, 4096, 12288
    for S in (2, 3, 4, 8, 16):
        assert dbd.gemm_workspace_bytes(dbd.DBD_BF16, M, N, K, 11, S) == 2 * 16 * S * 256 * 256 * 4
    assert dbd.gemm_workspace_bytes(dbd.DBD_BF16, M, N, K, 11, 1) == 0
    assert dbd.gemm_workspace_bytes(dbd.DBD_BF16, M, N, K, 3, 4) == 0
    assert dbd.gemm_workspace_bytes(dbd.DBD_BF16, 256, 256, 128, 11, 8) == 2 * 256 * 256 * 4


def test_gemm_split_plan_fits_workspace():
    """Split-K partials are sized by the same plan the launch uses: for every deep tile the
    workspace holds one fp32 tile per (output tile, split)."""
    for M, N, K in [(512, 4096, 4096), (512, 4096, 12288), (128, 2048, 4096), (16, 6144, 4096)]:
        for cfg in range(8, 19):
            b = dbd.gemm_workspace_bytes(dbd.DBD_BF16, M, N, K, cfg)
            assert b % 4 == 0
            if b:
                assert b >= 128 * 128 * 4 * 2


def test_gemm_override_validation():
    L = dbd.lib()
    assert L.dbd_gemm_override(5, -1, 0) == -1          # attention is not a GEMM stage
    assert L.dbd_gemm_override(4, 19, 0) == -1
    assert L.dbd_gemm_override(4, 10, 17) == -1
    # an override changes the planned split partials, and -1 / 0 restore the default
    sh = synth.workload("qwen3-8b").shape
    desc = dbd.model_desc(sh)
    base = dbd.draft_workspace_bytes(desc, 32, 16, 1, 64, 1, 0.0, 4096)
    dbd.gemm_override("gemm_down", 11, 8)
    try:
        # 2 x 16 output tiles of 256 x 256, 8 fp32 partials each: more than any default plan
        assert dbd.draft_workspace_bytes(desc, 32, 16, 1, 64, 1, 0.0, 4096) > base
    finally:
        dbd.gemm_override("gemm_down")
    assert dbd.draft_workspace_bytes(desc, 32, 16, 1, 64, 1, 0.0, 4096) == base


def test_verify_sample_validation():
    L = dbd.lib()
    fake = 1 << 20
    ws = dbd.verify_sample_workspace_bytes(4, 5, 6, 1000)
    assert ws > 0
    args = lambda **k: dict(dict(t=fake, d=fake, dr=fake, st=5, N=4, D=5, R=6, V=1000, tp=1.0,
                                 tq=1.0, seed=1, na=fake, b=fake, c=fake, f=None, w=fake,
                                 wb=ws), **k)
    call = lambda a: L.verify_sample(a["t"], a["d"], a["dr"], a["st"], a["N"], a["D"], a["R"],
                                     a["V"], a["tp"], a["tq"], a["seed"], a["na"], a["b"],
                                     a["c"], a["f"], a["w"], a["wb"], None)
    assert call(args(d=None)) == -1
    assert call(args(tp=0.0)) == -1
    assert call(args(tq=float("nan"))) == -1
    assert call(args(R=7)) == -2
    assert call(args(st=4)) == -2
    assert call(args(D=65, R=65)) == -5
    assert call(args(V=1 << 18)) == -1
    assert call(args(wb=ws - 1)) == -4
    assert call(args(w=fake + 16)) == -4


def test_context_path_switch_validation():
    L = dbd.lib()
    fake = 1 << 20
    for kw, code in ((dict(ctx_fusion=2), -1), (dict(mix_raw=3), -1),
                     (dict(ctx_shared_kv=-1), -1), (dict(ctx_fusion=1, mix_raw=1), -1)):
        d = _desc(**kw)
        out = ctypes.c_size_t(0)
        assert L.dbd_draft_workspace_bytes(ctypes.byref(d), 32, 16, 1, 64, 1, 0.0, 4096,
                                           ctypes.byref(out)) == code, kw
    # the fusion workspace holds one shared feature instead of one per draft layer
    mix = dbd.draft_workspace_bytes(_desc(), 32, 16, 1, 256, 1, 0.0, 4096)
    fc = dbd.draft_workspace_bytes(_desc("qwen3-8b-dflash"), 32, 16, 1, 256, 1, 0.0, 4096)
    assert fc < mix


def test_sample_top_p_validation():
    L = dbd.lib()
    fake = 1 << 20
    ws = dbd.sample_top_p_workspace_bytes(2, 3, 1000)
    assert ws > dbd.sample_workspace_bytes(2, 3, 1000)
    call = lambda T, p, wb=ws, w=fake: L.dbd_sample_top_p(fake, 2, 3, 1000, 4, T, p, 1, fake, w,
                                                          wb, None)
    assert call(0.0, 0.9) == -1
    assert call(1.0, 0.0) == -1
    assert call(1.0, float("nan")) == -1
    assert call(1.0, 0.9, wb=ws - 1) == -4
    assert call(1.0, 0.9, w=fake + 8) == -4


def test_refine_block_validation():
    L = dbd.lib()
    fake = 1 << 20
    ws = dbd.refine_workspace_bytes(2, 15, 1000)
    assert ws == dbd.sample_workspace_bytes(2, 15, 1000)

    def call(B=16, anchor=1, V=1000, mask=999, n=3, wb=ws, w=fake, lg=fake):
        return L.refine_block(lg, 2, B, anchor, V, mask, n, fake, fake, w, wb, None)

    assert call(lg=None) == -1
    assert call(anchor=2) == -1
    assert call(B=1) == -2 and call(B=65) == -2
    assert call(V=1 << 18, mask=5) == -2
    assert call(mask=1000) == -1 and call(mask=-1) == -1
    assert call(n=16) == -1 and call(n=-1) == -1
    assert call(wb=ws - 1) == -4
    assert call(w=fake + 8) == -4
