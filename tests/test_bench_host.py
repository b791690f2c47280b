"""Host checks of bench.py's accounting (no GPU).

The algorithmic bytes per pipeline are pinned to totals worked out by hand
from the byte model (x read once per real token, only routed rows of the
dispatch buffer and of y, index arrays read/written once) for each workload,
so a slip in the per-stage formulas changes every GB/s figure and fails
here."""
import os
import subprocess
import sys

import pytest

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# workload -> (routed slots V, bf16 pipeline bytes, MXFP4 pipeline bytes)
EXPECTED = {
    "tiny": (128, 199_760, 151_632),
    "mixtral_prefill": (14_000, 354_212_624, 269_988_624),
    "deepseek_v3_prefill": (32_768, 1_057_753_104, 712_771_600),
    "decode": (776, 27_356_208, 19_186_480),
    "large_prefill_stress": (491_520, 15_925_643_280, 10_750_920_720),
}


@pytest.mark.parametrize("name", sorted(EXPECTED))
def test_pipeline_bytes(name):
    v, bf16, mx = EXPECTED[name]
    w = workloads.BY_NAME[name]
    b = bench.stage_bytes(w, v)
    assert b["mask"] + b["indices"] + b["dispatch_bf16"] + b["combine"] == bf16
    assert b["mask"] + b["indices"] + b["dispatch_mxfp4"] + b["combine"] == mx


def test_routed_slots_of_the_workloads():
    """V = real tokens x top_k for every workload (padding rows only are unrouted)."""
    for name, (v, _, _) in EXPECTED.items():
        w = workloads.BY_NAME[name]
        assert w.real_tokens * w.top_k == v


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def test_source_digest_ignores_comments(tmp_path, monkeypatch):
    """Counters stay valid across comment edits and go stale on a code edit."""
    import shutil
    csrc = tmp_path / "expert_grouping_dispatch_amd" / "csrc"
    csrc.mkdir(parents=True)
    real = os.path.join(ROOT, "expert_grouping_dispatch_amd", "csrc")
    for f in ("combine.hip", "rows.h", "common.h"):
        shutil.copy(os.path.join(real, f), csrc / f)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    d0 = bench.source_digest("k_combine")
    text = (csrc / "combine.hip").read_text()
    (csrc / "combine.hip").write_text("// a new comment\n" + text.replace("\n", "\n  ", 3))
    assert bench.source_digest("k_combine") == d0
    (csrc / "combine.hip").write_text(text.replace("kBatch = 8", "kBatch = 4"))
    assert bench.source_digest("k_combine") != d0


def test_kernel_labels_follow_the_launch_rule():
    """The roofline label names the kernel the library launches: the
    loop-free bf16 dispatch for top_k <= 8, the loop-free combine below
    1 GiB of routed y rows, whole-row combine above, and the
    four-lanes-per-block MXFP4 kernel from 256 MiB of output with
    top_k <= 8."""
    by = workloads.BY_NAME
    stress, decode = by["large_prefill_stress"], by["decode"]
    assert bench.kernel_of_stage("dispatch_bf16", stress) == "k_dispatch_bf16_parts"
    assert bench.kernel_of_stage("combine", stress) == "k_combine"
    assert bench.kernel_of_stage("combine", decode) == "k_combine_parts"
    assert bench.kernel_of_stage("dispatch_mxfp4", decode) == "k_dispatch_mxfp4"
    assert bench.kernel_of_stage("dispatch_mxfp4", stress) == "k_dispatch_mxfp4_quad"
    assert bench.kernel_of_stage("dispatch_mxfp4", workloads.scaled(stress, top_k=9)) == "k_dispatch_mxfp4"
    wide = workloads.scaled(decode, top_k=9)
    assert bench.kernel_of_stage("dispatch_bf16", wide) == "k_dispatch_bf16"
    assert bench.kernel_of_stage("combine", wide) == "k_combine"
    assert bench.source_digest("k_combine_parts") == bench.source_digest("k_combine")
    assert bench.source_digest("k_dispatch_bf16_parts") == bench.source_digest("k_dispatch_bf16")
    # the two dispatch formats live in separate sources: a change to one
    # leaves the other's counters current
    assert bench.source_digest("k_dispatch_bf16") != bench.source_digest("k_dispatch_mxfp4")


def test_stress_counter_profiles_are_current():
    """The committed rocprofv3 counter summaries of the three row kernels on
    the stress workload were taken on the current kernel sources, so the
    bench reports their measured HBM bytes (and those stay within 2% of the
    algorithmic bytes: nothing is re-read)."""
    w = workloads.BY_NAME["large_prefill_stress"]
    n_routed = w.real_tokens * w.top_k
    bts = bench.stage_bytes(w, n_routed)
    for stage in bench.ROW_STAGES:
        counted = bench.read_traffic(bench.kernel_of_stage(stage, w), w.name)
        assert counted is not None, stage
        assert 1.0 <= counted / bts[stage] < 1.02, (stage, counted / bts[stage])
