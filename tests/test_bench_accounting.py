"""The benchmark's algorithmic byte accounting, checked on the CPU.

The headline GB/s is bytes per layer-step divided by time, so the byte count
is checked against totals worked out by hand from the layer shapes alone: the
predictor's two matrices and bias, the selected neurons' rows (gate, up, down;
int4 rows with their fp16 group scales) and fp32 biases, the dense
pre-activation matrix in exact mode, x, y and the index list.  The selected
counts are the expected active neurons of each workload, E|M| = sum over
neurons of 1 - (1 - p_i)^B under the synthetic firing law, and they are pinned
here too.
"""

import numpy as np
import pytest

import bench
from synth import config_by_name
from synth.layers import firing_probs

# (workload, mode, batch, expected active count, MB per layer-step), to two decimals
HAND_TOTALS = [
    ("toy", "predicted", 1, 205, 1.51),
    ("llama7b", "predicted", 1, 1101, 58.06),
    ("llama7b", "exact", 1, 1101, 108.28),
    ("llama7b", "dense", 1, 11008, 270.59),
    ("opt30b", "predicted", 1, 1434, 114.67),
    ("opt30b", "exact", 1, 1434, 431.75),
    ("falcon40b", "predicted", 1, 2621, 108.24),
    ("falcon40b", "exact", 1, 2621, 163.26),
    ("llama70b", "predicted", 1, 2867, 216.61),
    ("llama70b", "predicted", 4, 6943, 417.10),
    ("llama70b", "predicted", 16, 15218, 824.31),
    ("llama70b", "dense", 1, 28672, 1409.43),
]


@pytest.mark.parametrize("name,mode,B,count,mb", HAND_TOTALS)
def test_step_bytes_match_hand_totals(name, mode, B, count, mb):
    got = bench.step_bytes(config_by_name(name), mode, B, count) / 1e6
    assert abs(got - mb) <= max(0.01, 1e-3 * mb), f"{name} {mode} B={B}: {got:.2f} MB, by hand {mb:.2f} MB"


@pytest.mark.parametrize("name,B,count", [
    ("toy", 1, 205), ("llama7b", 1, 1101), ("opt30b", 1, 1434), ("falcon40b", 1, 2621),
    ("llama70b", 1, 2867), ("llama70b", 4, 6943), ("llama70b", 16, 15218),
])
def test_expected_active_counts(name, B, count):
    p = firing_probs(config_by_name(name), 0)
    e = float(np.sum(1.0 - (1.0 - p) ** B))
    assert abs(e - count) <= max(1.0, 2e-3 * count), f"{name} B={B}: E|M| = {e:.1f}, expected about {count}"


@pytest.mark.parametrize("name,mode,B,path", [
    ("llama7b", "predicted", 1, "split"), ("falcon40b", "predicted", 1, "split"), ("llama7b", "exact", 1, "split"),
    ("llama70b", "dense", 1, "split"), ("llama70b", "predicted", 16, "batched"), ("llama7b", "exact", 4, "batched"),
    ("llama70b", "exact", 64, "batched"), ("llama70b", "dense", 32, "batched"),
    ("toy", "predicted", 1, "vector"), ("toy", "exact", 1, "vector")])
def test_phase_bytes_cover_the_step(name, mode, B, path):
    """The per-kernel algorithmic bytes (the roofline's numerator) add up to the step's bytes
    plus exactly the hand-offs between kernels: x read by a second kernel, h written and read
    back (predicted mode), and the mask bits written and read again (by the down kernel of a
    batch or of the one-token split path, or by the finish kernel)."""
    cfg = config_by_name(name)
    count = 2000 if mode != "dense" else cfg.d_ffn
    head = ("pred_hidden",) if mode == "predicted" else ()
    phases = head + {"split": ("group", "down"), "batched": ("group", "down", "finish"),
                     "vector": ("group", "finish")}[path]
    total = sum(bench.phase_bytes(cfg, mode, ph, B, count, phases) for ph in phases)
    step = bench.step_bytes(cfg, mode, B, count)
    if mode == "dense":
        handoff = 0.0 if path == "split" else cfg.d_ffn / 8
    else:
        handoff = cfg.d_ffn / 8 * (2 if path != "vector" else 1)
    if mode == "predicted":
        handoff += B * cfg.d_model * bench.esize(cfg.act_dtype) + 2 * B * cfg.rank * 4
    assert abs(total - (step + handoff)) <= 1, (total, step, handoff)


def test_counter_calibration_uses_only_the_calibration_copy(tmp_path):
    """HBM counters are scaled by what they read for the 256 MiB calibration copy.  Other copy
    kernels in the same process (1 GiB device copies, weight uploads) must not enter the scale."""
    def write_csv(path, counter, rows):
        with open(path, "w") as f:
            f.write("Kernel_Name,Counter_Name,Counter_Value\n")
            for name, value in rows:
                f.write(f'"{name}",{counter},{value}\n')

    copy, kern = "__amd_rocclr_copyBuffer", "void pik::k_act<1, 16, 0, 8>(pik::GroupArgs, float*)"
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    # calibration copy: FETCH_SIZE reads half of 256 MiB, WRITE_SIZE all of it (KiB); a 1 GiB copy
    # reads four times as much; the kernel fetched 1000 KiB and wrote 10 KiB per dispatch
    write_csv(fetch, "FETCH_SIZE", [(copy, 131072), (copy, 131072), (copy, 524288), (kern, 1000), (kern, 1000)])
    write_csv(write, "WRITE_SIZE", [(copy, 262144), (copy, 1048576), (kern, 10), (kern, 10)])
    res = bench.summarize_pmc(str(fetch), str(write), 256, "w", 1)
    assert res["fetch_scale"] == pytest.approx(2.0) and res["write_scale"] == pytest.approx(1.0)
    rec = res["kernels"]["w/group"]
    assert rec["dispatches"] == 2
    assert rec["fetch_bytes_per_launch"] == 2 * 1000 * 1024 and rec["write_bytes_per_launch"] == 10 * 1024


def test_bench_refuses_more_than_one_gpu():
    """The path runs on one GPU: --gpus N > 1 exits with status 2 and says so, before touching a GPU."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr or "one MI355X" in res.stderr
    assert res.stdout == ""


def test_budget_rank_policy():
    """The per-layer rank policy: the largest multiple of 64 whose predictor bytes fit the budget,
    worked by hand for the Llama2-70B shape (expected active 2867 neurons of 3 x 16 KB rows)."""
    cfg = config_by_name("llama70b")
    p = firing_probs(cfg, 0)
    active = bench.expected_active(p, 1) * (3 * 8192 * 2 + 4)
    per_rank = (8192 + 28672) * 2          # predictor bytes per unit of rank, plus 4 n for b_p
    for frac in (0.03, 0.2, 0.35, 1.0):
        r = bench.budget_rank(cfg, p, 1, frac)
        assert r % 64 == 0 and 64 <= r <= 1024
        fits = lambda rr: rr * per_rank + 4 * 28672 <= frac * active
        assert r == 64 or fits(r)
        assert r == 1024 or not fits(r + 64)
    assert bench.budget_rank(cfg, p, 1, 0.03) == 64        # the pages' "under 3 %" leaves the smallest rank
    assert bench.budget_rank(cfg, p, 1, 1.0) == 1024


@pytest.mark.parametrize("name", ["llama7b", "falcon40b", "llama70b"])
def test_phase_bytes_with_a_hot_head(name):
    """With a hot head the group kernel no longer reads the head's P2 rows and b_p, and the kernels
    still add up to the step (which no longer reads them either) plus the hand-offs."""
    cfg = config_by_name(name)
    count, n_hot = 3000, 704
    phases = ("pred_hidden", "group", "down")
    total = sum(bench.phase_bytes(cfg, "predicted", ph, 1, count, phases, n_hot) for ph in phases)
    step = bench.step_bytes(cfg, "predicted", 1, count, n_hot)
    handoff = cfg.d_ffn / 8 * 2 + cfg.d_model * 2 + 2 * cfg.rank * 4
    assert abs(total - (step + handoff)) <= 1, (total, step, handoff)
    saved = bench.step_bytes(cfg, "predicted", 1, count) - step
    assert saved == n_hot * (cfg.rank * 2 + 4)


def test_mode_run_past_16_tokens():
    """A PREDICTED call of more than 16 tokens runs as EXACT_RELU; other modes and batches run as asked."""
    assert bench.mode_run("predicted", 1) == "predicted"
    assert bench.mode_run("predicted", 16) == "predicted"
    assert bench.mode_run("predicted", 17) == "exact"
    assert bench.mode_run("predicted", 64) == "exact"
    assert bench.mode_run("dense", 64) == "dense"
    assert bench.mode_run("exact", 32) == "exact"


def test_stored_counters_only_for_the_profiled_configuration():
    """Counter bytes were taken on each workload as configured; a changed rank, a rank policy or a
    hot set reads other predictor bytes, so the bench line's traffic is then null."""
    assert bench.counters_apply(0, "fixed", 0.0)
    assert not bench.counters_apply(256, "fixed", 0.0)
    assert not bench.counters_apply(0, "budget:0.03", 0.0)
    assert not bench.counters_apply(0, "fixed", 0.99)
