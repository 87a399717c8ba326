"""Checks of bench.py's contract.  On the host: more than one GPU is refused
before anything touches a device, the committed HBM-traffic summaries belong
to the attention kernel's current source (so that the bench line's
`roofline.traffic` is a measurement of the code that runs), the kernel label
follows the planner's rule, and --batch builds the batch its spec names.  On
the GPU: bench.py end to end on small workloads prints one line with the
contract's fields."""
import json
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_traffic_summary_matches_the_kernel_source():
    with open(bench.PMC_SUMMARY) as f:
        s = json.load(f)
    assert s["kernel_source_hash"] == bench.kernel_source_hash()
    got = bench.measured_traffic(s["config"], 1)
    assert got is not None and got > 0
    # the traffic is the algorithmic bytes of config 4 within a few percent
    alg = ((2 * 8192 + 4 * 512) * 128 * 2 + 4 * 512) * 16 * 16
    assert abs(got / alg - 1.0) < 0.05


def test_every_committed_traffic_summary_is_current():
    """Each per-configuration summary that is committed names its own
    configuration and the kernel source that runs now."""
    found = 0
    for config, path in bench.PMC_SUMMARIES.items():
        if not os.path.exists(path):
            continue
        found += 1
        with open(path) as f:
            s = json.load(f)
        assert s["config"] == config
        assert s["kernel_source_hash"] == bench.kernel_source_hash()
        assert bench.measured_traffic(config, 1) == s["hbm_bytes_per_launch"] > 0
    assert found >= 1
    assert bench.measured_traffic("config9", 1) is None


@pytest.mark.parametrize("config,profile", [
    (2, "attn_bf16_d64_config2.md"), (3, "attn_bf16_d64_config3.md"),
    (4, "attn_bf16_d128_config4.md"), (5, "attn_bf16_d128_config5.md")])
def test_kernel_label_is_the_kernel_the_profile_traced(config, profile):
    """The bench line's kernel name follows the library's workgroup-shape
    rule; the committed kernel trace of each configuration shows which
    kernel the library actually launched."""
    from prefix_reuse_attention_amd import workloads as W
    with open(os.path.join(ROOT, "profiles", profile)) as f:
        traced = re.findall(r'^"void bat::(attn_bf16_\w+<[^>]*>)\(', f.read(), flags=re.M)
    assert len(set(traced)) == 1
    label = bench.bf16_kernel_label(W.make_config(config))
    # the trace names every template argument, the label the first ones
    assert traced[0].startswith(label[:-1])


def test_source_hash_ignores_comments(tmp_path, monkeypatch):
    """The hash covers code only: a comment or blank line edit keeps it."""
    csrc = tmp_path / "prefix_reuse_attention_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in ("attn_bf16.hip", "common.h"):
        with open(os.path.join(ROOT, "prefix_reuse_attention_amd", "csrc", f)) as fh:
            (csrc / f).write_text(fh.read())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash()
    (csrc / "common.h").write_text((csrc / "common.h").read_text() + "\n// a note\n\n/* more */\n")
    assert bench.kernel_source_hash() == h0
    (csrc / "common.h").write_text((csrc / "common.h").read_text() + "\nconstexpr int kX = 1;\n")
    assert bench.kernel_source_hash() != h0


def test_batch_spec():
    """--batch builds the batch its spec names: fixed or uniformly drawn
    lengths within their bounds, item prefixes in whole 4-token items, the
    same batch for the same seed, and an error for an unknown key."""
    from prefix_reuse_attention_amd import workloads as W
    wl = bench.batch_from_spec("B=6,H=2,D=64,n_p=100:900,n_s=257:512,mode=mixed,seed=5")
    assert (wl.B, wl.H, wl.D) == (6, 2, 64)
    assert ((wl.n_s >= 257) & (wl.n_s <= 512)).all()
    assert ((wl.n_p >= 96) & (wl.n_p <= 900)).all()
    assert (wl.n_p[wl.mode == W.ITEM] % W.ITEM_TOKENS == 0).all()
    again = bench.batch_from_spec("B=6,H=2,D=64,n_p=100:900,n_s=257:512,mode=mixed,seed=5")
    assert (again.n_s == wl.n_s).all() and (again.n_p == wl.n_p).all()
    assert (again.mode == wl.mode).all()
    fixed = bench.batch_from_spec("B=3,H=1,D=128,n_p=8192,n_s=300")
    assert fixed.n_p.tolist() == [8192] * 3 and fixed.n_s.tolist() == [300] * 3
    assert (fixed.mode == W.USER).all()
    assert bench.measured_traffic(fixed.name, 1) is None
    with pytest.raises(SystemExit):
        bench.batch_from_spec("B=3,rows=4")
    with pytest.raises(SystemExit):
        bench.batch_from_spec("B=3,D128")


def _bench_line(*args):
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), *args],
                       capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    return json.loads(lines[0])


@pytest.mark.gpu
@pytest.mark.parametrize("args,kernel", [
    (("--config", "1"), "attn_f32_kernel<32>"),
    (("--batch", "B=2,H=2,D=128,n_p=200,n_s=300"), "attn_bf16_pp_kernel<128, false>"),
    (("--batch", "B=3,H=2,D=64,n_p=64:400,n_s=20:90,mode=mixed,seed=4"),
     "attn_bf16_kernel<64, 4, false>")])
def test_bench_line_on_the_gpu(gpu_ready, args, kernel):
    """bench.py end to end on small workloads: one JSON line with the
    contract's fields, the timed steps and the per-call pass, and the kernel
    the planner's rule names."""
    d = _bench_line(*args, "--steps", "3", "--warmup", "1", "--no-cpu-baseline")
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert d["roofline"]["kernel"] == kernel
    assert d["roofline"]["achieved"] > 0 and 0 <= d["roofline"]["frac"] < 1
    pc = d["per_call_ms"]
    assert pc["calls"] == 3 and 0 < pc["min"] <= pc["median"] <= pc["p90"]
