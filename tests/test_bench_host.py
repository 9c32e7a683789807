"""Host-side checks of the bench's bookkeeping (CPU only): the stage-to-kernel lookups that tie
the timed stages to the committed counter summaries, and the source hash that dates them."""
import json

import pytest

import bench


def _kernel_names(path):
    return list(json.load(open(path))["kernels"])


@pytest.mark.parametrize("path", [bench.TRAFFIC_FILE, bench.COUNTERS_FILE])
def test_every_looked_up_stage_finds_its_kernel(path):
    """Each stage whose traffic or MFMA counters the bench line reports maps to one library
    kernel of the committed summary (a renamed kernel would otherwise report null)."""
    names = _kernel_names(path)
    for stage in list(bench.STAGE_EPILOGUE) + list(bench.STAGE_KERNEL):
        assert len(bench.stage_kernels(stage, names)) == 1, (stage, path)


def test_gemm_epilogue_reads_the_template_argument():
    g = bench.gemm_epilogue
    assert g("void dbd::gemm_w8r_kernel<192, 4, 4, false>(dbd::GemmArgs, dbd::EpiArgs)") == 4
    assert g("void dbd::gemm_w8r_kernel<256, 5, 2, true>(dbd::GemmArgs, dbd::EpiArgs)") == 5
    assert g("void dbd::gemm_big_kernel<128, 128, 6, 3, true>(dbd::GemmArgs, dbd::EpiArgs)") == 3
    assert g("void dbd::gemm_bf16_kernel<64, 128, 3, 1, false>(dbd::GemmArgs, dbd::EpiArgs)") == 1
    # the split-K reduction carries the epilogue too, but is not the stage's main kernel
    assert g("void dbd::gemm_reduce_kernel<256, 128, 4, 2, 2, false>(dbd::GemmArgs, "
             "dbd::EpiArgs)") is None
    assert g("dbd::attn_stream_combine_kernel(dbd::AttnArgs, int)") is None


def test_attention_lookup_takes_the_main_kernel_only():
    names = ["void dbd::attn_stream_kernel<128, true, 1>(dbd::AttnArgs)",
             "dbd::attn_stream_combine_kernel(dbd::AttnArgs, int)",
             "dbd::attn_plan_kernel(int const*, int, int, int, int, dbd::AttnPlan*, int*, long*)"]
    assert bench.stage_kernels("attn", names) == names[:1]


def test_source_hash_ignores_comments_only(tmp_path):
    src = {"a": "int x; // one\n/* two\n three */ int y;\n",
           "b": "int x; // another\n/* other */ int y;\n",
           "c": "int x; int z;\n"}
    h = {}
    for k, text in src.items():
        d = tmp_path / k
        d.mkdir()
        (d / "k.hip").write_text(text)
        h[k] = bench.kernel_source_hash(str(d))
    assert h["a"] == h["b"]
    assert h["a"] != h["c"]
