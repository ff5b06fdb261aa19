"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the byte and
flop accounting tables, and the oracle baseline's unit."""
import json
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import race_inputs as ri  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_every_streaming_kernel_has_a_byte_count():
    """Each kernel the library times over token rows appears in the
    accounting table, so the roofline line never prices it at zero bytes."""
    src = open(os.path.join(ROOT, "linear_attention_soft_amd", "csrc", "race_api.cpp")).read()
    timed = set(re.findall(r'ProfScope ps\(s, "(race_[a-z_]+)"\)', src))
    # race_copy_rows pads token rows for head dims between the compiled ones
    # (never at the workloads' d = 64 and 128)
    no_rows = {"race_bank_finalize", "race_seg_scan", "race_dbeta_finalize", "race_dw_partial",
               "race_dw_finalize", "race_decode", "race_decode_prefill", "race_copy_rows"}
    assert timed - no_rows <= set(bench.ROW_PASSES), timed - no_rows - set(bench.ROW_PASSES)
    # the whole step reads or writes 11 row tensors: forward 4, backward 7
    nc_fwd = bench.ROW_PASSES["race_bucket_reduce"] + bench.ROW_PASSES["race_readout_norm"]
    nc_bwd = bench.ROW_PASSES["race_bwd_q"] + bench.ROW_PASSES["race_bwd_kv"]
    assert (nc_fwd, nc_bwd) == (4, 7)


def test_causal_flop_counts():
    L, P, d = 4, 6, 128
    LR = L << P
    assert bench.causal_flops("race_causal_dk", L, P, d) == 2 * LR * d + 2 * LR * (d + 1) + 2 * L * P * d
    assert bench.causal_flops("race_causal_fwd", L, P, d) == 4 * LR * (d + 1)
    assert bench.causal_flops("race_bwd_kv", L, P, d) is None


def test_cpu_baseline_rate_counts_all_heads():
    """The oracle sample covers one head; a metric token carries all H, so the
    reported rate is the sample's tokens over H times its time."""
    w = ri.WORKLOADS[2].with_size(N=64, B=1, H=4)
    inp = ri.make_inputs(w, device="cpu", with_grad_out=True)
    rec = bench.cpu_baseline(inp, w, 64)
    assert rec["kind"] == "oracle" and rec["unit"] == "tokens/s" and rec["cores"] >= 1
    m = re.search(r"(\d+) pass\(es\) in ([0-9.]+) s", rec["sample"])
    reps, t = int(m.group(1)), float(m.group(2))
    assert "fwd fp64" in rec["sample"] and "fwd+bwd" not in rec["sample"]
    assert t >= 1.0   # short samples repeat until a second has passed
    assert rec["value"] == pytest.approx(64 * reps / (4 * t), rel=0.02)
    json.dumps(rec)


def test_cpu_baseline_sample_is_sized_by_a_probe():
    """Without a sample length the probe sizes the sample for the target time,
    within the workload's length."""
    w = ri.WORKLOADS[1]
    inp = ri.make_inputs(w, device="cpu")
    rec = bench.cpu_baseline(inp, w, target_s=0.5)
    # workload 1 is one sequence of 1024 tokens: the sample is the whole workload
    assert rec["sample"].startswith("the whole workload") and rec["extrapolated"] is False
    w2 = ri.WORKLOADS[2].with_size(N=300, B=1, H=2)
    rec2 = bench.cpu_baseline(ri.make_inputs(w2, device="cpu"), w2, target_s=0.3)
    assert rec2["extrapolated"] is True and "extrapolated" in rec2["sample"]
    assert re.search(r"first \d+ of 300 tokens", rec2["sample"])
