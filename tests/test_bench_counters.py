"""Host logic of bench.py's counter summaries, on counter files written here
in the layout rocprofv3 --output-format csv uses (no GPU, no profiler)."""

import csv
import json
import os

import pytest

import bench

FAMILY_KERNEL = {"compress": "void bd::(anonymous namespace)::compress_rows_kernel<true>(x)",
                 "decode": "void bd::(anonymous namespace)::linear_decode_ring_kernel<1, 8, 2>(x)",
                 "multi": "void bd::(anonymous namespace)::linear_multi_pairs_kernel<2>(x)",
                 "prefill": "void bd::(anonymous namespace)::prefill_pc_kernel<false>(x)",
                 "reconstruct": "void bd::(anonymous namespace)::reconstruct_kernel<2>(x)"}


SEP = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<unsigned char>>(x)"


def write_run(d, workload, n, counters, value_of, launches=1):
    """A fake run: set-up launches, then a separator, n calls per block (each
    of `launches` launches) and a separator after each block, then n
    calibration launches; value_of(block, counter, r) gives each counter's
    value per call, split evenly over the call's launches."""
    os.makedirs(d, exist_ok=True)
    blocks, _ = bench.counter_plan(workload)
    rows, did = [], 1
    for k in (FAMILY_KERNEL["compress"], SEP):
        for c in counters:
            rows.append((did, k, c, 1.0))
        did += 1
    for name, fam, _ in blocks:
        for r in range(n):
            for _ in range(launches):
                for c in counters:
                    rows.append((did, FAMILY_KERNEL[fam], c, value_of(name, c, r) / launches))
                did += 1
        for c in counters:
            rows.append((did, SEP, c, 1.0))
        did += 1
    for c in counters:   # the calibration buffer's zero fill
        rows.append((did, "void at::native::FillFunctor<c10::BFloat16>(x)", c, 5.0))
    did += 1
    for r in range(n):
        for c in counters:
            rows.append((did, "void at::native::neg_kernel(x)", c, value_of("calib", c, r)))
        did += 1
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writerows(rows)


@pytest.mark.parametrize("workload,launches", [(w, 1) for w in bench.COUNTER_WORKLOADS]
                         + [("layer70b_prefill", 2)])
def test_traffic_scaled_by_calibration(tmp_path, monkeypatch, workload, launches):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    os.makedirs(bench.PROFILES)
    n = 3
    blocks, groups = bench.counter_plan(workload)
    alg = {b: v for b, _, v in blocks}
    calib_kib = bench.CALIB_BYTES / 1024 / 2   # the counter reads half the true bytes

    def fetch(name, c, r):
        return calib_kib if name == "calib" else alg[name] / 1024 / 2 * (1 + 0.1 * (r - 1))

    def write(name, c, r):
        return calib_kib if name == "calib" else 1000.0

    write_run(tmp_path / "f", workload, n, ["FETCH_SIZE"], fetch, launches)
    write_run(tmp_path / "w", workload, n, ["WRITE_SIZE"], write, launches)
    res, per = bench.summarize_counters(str(tmp_path / "f"), str(tmp_path / "w"), workload, n)
    assert per["FETCH_SIZE"]["factor"] == pytest.approx(2.0)
    for b in alg:
        assert res[b]["hbm_bytes"] == pytest.approx(alg[b] + 2 * 1000 * 1024, rel=1e-9)
    bench.write_counter_profiles(res, per, workload, n)
    for fam, (labels, _) in groups.items():
        rec = json.load(open(os.path.join(bench.PROFILES, f"{fam}_{workload}_pmc.json")))
        assert rec["hbm_bytes_per_launch"] == sum(res[l]["hbm_bytes"] for l in labels)
        assert rec["sources_digest"] == bench.sources_digest(bench.KERNEL_SOURCES[fam])
    assert os.path.exists(os.path.join(bench.PROFILES, f"counters_{workload}.md"))


def test_launch_count_not_a_multiple_of_calls_is_refused(tmp_path):
    d = tmp_path / "f"
    write_run(d, "proj_4096", 2, ["FETCH_SIZE"], lambda b, c, r: 1.0)
    p = d / "run_counter_collection.csv"
    lines = p.read_text().splitlines(keepends=True)
    # drop the first decode launch: that block then holds 1 launch for 2 calls
    i = next(k for k, l in enumerate(lines) if "linear_decode_" in l)
    p.write_text("".join(lines[:i] + lines[i + 1:]))
    with pytest.raises(SystemExit):
        bench.summarize_counters(str(d), str(d), "proj_4096", 2)


def test_block_with_a_foreign_kernel_is_refused(tmp_path):
    d = tmp_path / "f"
    write_run(d, "layer70b_multi", 2, ["FETCH_SIZE"], lambda b, c, r: 1.0)
    p = d / "run_counter_collection.csv"
    text = p.read_text().replace("linear_multi_pairs_kernel<2>(x),FETCH_SIZE,1.0\n",
                                 "prefill_pc_kernel<false>(x),FETCH_SIZE,1.0\n", 1)
    p.write_text(text)
    with pytest.raises(SystemExit):
        bench.summarize_counters(str(d), str(d), "layer70b_multi", 2)


def test_sq_summary_derives_from_one_run(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    os.makedirs(bench.PROFILES)
    vals = {"GRBM_GUI_ACTIVE": 8000.0, "SQ_VALU_MFMA_BUSY_CYCLES": 512000.0,
            "SQ_WAIT_ANY": 30.0, "SQ_WAVE_CYCLES": 60.0}
    write_run(tmp_path / "a", "layer70b_prefill", 2, list(vals), lambda b, c, r: vals[c])
    bench.summarize_pmc([str(tmp_path / "a")], "layer70b_prefill", 2)
    text = open(os.path.join(bench.PROFILES, "sq_counters_layer70b_prefill.md")).read()
    # 512000 / (1024 SIMDs x 1000 clocks) = 50%; 30 / 60 = 50%
    assert "| MFMA pipe busy per SIMD" in text and "50.0%" in text
    assert "--counter-pass --workload layer70b_prefill" in text
