"""Host logic of bench.py and of the profile summaries (no GPU needed): the
one-GPU refusal, the per-role work and roofline arithmetic, the choice of
the dominant kernel, and the rule that counter traffic is reported only for
the GEMM sources it was measured on."""
import os
import subprocess
import sys

import pytest

import bench
import synth
from routing_grouped_gemm_router_amd import rocprof_summary as rps

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""            # no JSON line


def _gemm_flops_by_shape(w):
    """2 * rows * N * K of every GEMM role, from the operand shapes of the
    layer (x [R, d], W1 [2h, d], H' [R, h], W2 [d, h]), summed per expert."""
    counts = [w.R // w.E] * w.E
    counts[0] += w.R - sum(counts)
    f = {}
    f["gemm1_swiglu"] = sum(2 * c * (2 * w.h) * w.d for c in counts)     # x . W1^T
    f["gemm2"] = sum(2 * c * w.d * w.h for c in counts)                  # H' . W2^T
    f["gemm2_dgrad_swiglu"] = sum(2 * c * w.h * w.d for c in counts)     # dy . W2
    f["gemm2_wgrad"] = sum(2 * w.d * w.h * c for c in counts)            # dy^T . H'
    f["gemm1_dgrad"] = sum(2 * c * w.d * (2 * w.h) for c in counts)      # dAB . W1
    f["gemm1_wgrad"] = sum(2 * (2 * w.h) * w.d * c for c in counts)      # dAB^T . x
    return f


@pytest.mark.parametrize("name", ["e128_bf16", "e128_mxfp8", "e8_bf16_fwd"])
def test_role_flops_match_the_operand_shapes(name):
    w = synth.WORKLOADS[name]
    work = bench.role_work(w)
    for role, fl in _gemm_flops_by_shape(w).items():
        assert work[role][0] == fl, role
    # the layer's flops are the six GEMM roles
    assert w.fwd_bwd_flops() == sum(_gemm_flops_by_shape(w).values())


def test_role_bytes_of_the_row_movers():
    w = synth.WORKLOADS["e128_bf16"]
    work = bench.role_work(w)
    T, d, R = w.T, w.d, w.R
    assert work["permute"][1] == 2 * T * d + 2 * R * d           # each token read, k rows written
    assert work["unpermute_bwd"][1] == 2 * R * d + 2 * T * d + 4 * T * w.k


def test_role_table_fractions():
    w = synth.WORKLOADS["e128_bf16"]
    work = bench.role_work(w)
    times = {"gemm1_swiglu": 0.640, "gemm1_wgrad": 0.900, "permute": 0.056}
    t = bench.role_table(w, times)
    g = t["gemm1_swiglu"]
    assert g["tflops"] == pytest.approx(work["gemm1_swiglu"][0] / 0.640e-3 / 1e12)
    assert g["frac_mfma"] == pytest.approx(g["tflops"] / bench.PEAK_BF16_TFLOPS)
    assert g["bound"] == "mfma" and g["frac_roof"] == pytest.approx(g["frac_mfma"])
    wg = t["gemm1_wgrad"]                # 2 GiB of fp32 dW1: bound by HBM
    assert wg["bound"] == "hbm" and wg["frac_roof"] == pytest.approx(wg["frac_hbm"])
    assert wg["gbps"] == pytest.approx(work["gemm1_wgrad"][1] / 0.900e-3 / 1e9)
    p = t["permute"]
    assert "tflops" not in p and p["bound"] == "hbm"


def test_dominant_roofline_is_the_longest_gemm_launch():
    w = synth.WORKLOADS["e128_bf16"]
    times = {"permute": 2.0, "gemm1_swiglu": 0.640, "gemm2": 0.350, "gemm1_wgrad": 0.900,
             "gemm2_wgrad": 0.450}
    roles = bench.role_table(w, times)
    r = bench.dominant_roofline(w, roles, traffic=2.8e9)
    assert "gemm1_wgrad" in r["kernel"] and "gg_ws" in r["kernel"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == bench.PEAK_HBM_GBS
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"])
    assert r["traffic"] == 2.8e9
    times["gemm1_swiglu"] = 1.5           # now the forward GEMM is the longest: MFMA-bound
    r = bench.dominant_roofline(w, bench.role_table(w, times), traffic=None)
    assert "gemm1_swiglu" in r["kernel"] and r["unit"] == "TFLOP/s"
    assert r["peak"] == bench.PEAK_BF16_TFLOPS and r["traffic"] is None


def test_traffic_only_for_the_sources_it_was_measured_on(tmp_path):
    md = tmp_path / "x_pmc.md"
    md.write_text("# t\n\ntraffic_bytes_per_launch = 1.5e+09\ngemm_source_hash = deadbeef00000000\n")
    t, h = rps.read_traffic(str(md))
    assert t == 1.5e9 and h == "deadbeef00000000"
    assert h != rps.gemm_source_hash()     # a stale summary: the bench reports null
    md.write_text("# t\n\ntraffic_bytes_per_launch = 1.5e+09\n")
    assert rps.read_traffic(str(md)) is None
    assert rps.read_traffic(str(tmp_path / "missing.md")) is None


def test_committed_counter_summaries_name_their_sources():
    prof = os.path.join(ROOT, "profiles")
    pmc = [f for f in os.listdir(prof) if f.endswith("_pmc.md")]
    assert pmc
    for f in pmc:
        r = rps.read_traffic(os.path.join(prof, f))
        assert r is not None and len(r[1]) == 16, f


def test_role_table_carries_median_and_min():
    w = synth.WORKLOADS["e128_bf16"]
    st = bench.StageTimes()
    st["gemm2"] = 0.350
    st.spread["gemm2"] = (0.348, 0.341)
    r = bench.role_table(w, st)["gemm2"]
    assert r["us"] == pytest.approx(350.0)
    assert r["us_median"] == pytest.approx(348.0) and r["us_min"] == pytest.approx(341.0)
    assert "us_median" not in bench.role_table(w, {"gemm2": 0.350})["gemm2"]


def test_counter_tables_of_the_row_movers(tmp_path):
    """The multi-kernel summary: copy-scaled bytes per launch, the n-th of
    every p launches of a shared name, and the hash of the row sources."""
    import csv

    def write(d, counter, rows):
        d.mkdir()
        with open(d / "run_counter_collection.csv", "w", newline="") as f:
            w = csv.DictWriter(f, ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
            w.writeheader()
            for i, (name, kib) in enumerate(rows):
                for half in (0.5, 0.5):              # two counter instances per dispatch
                    w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter,
                                "Counter_Value": kib * half})
    step = [("moe::permute_rows16<4>", 100.0), ("moe::mx_quant_cols_bf16<true>", 10.0),
            ("moe::mx_quant_cols_bf16<true>", 20.0), ("__amd_rocclr_copyBuffer", 512.0)]
    write(tmp_path / "f", "FETCH_SIZE", step)
    write(tmp_path / "w", "WRITE_SIZE", [(n, 2 * v) for n, v in step])
    md = rps.counters(str(tmp_path / "f"), str(tmp_path / "w"),
                      ["dispatch=permute_rows16", "second=mx_quant_cols_bf16<true>#1/2"],
                      1024 * 1024, "t", "cf", "cw")
    rows = {l.split("|")[1].strip(): l.split("|") for l in md.splitlines() if l.startswith("| d") or l.startswith("| s")}
    # FETCH: the copy of 1 MiB reads 512 KiB -> x2; WRITE: 1 MiB -> x1
    assert float(rows["dispatch"][4]) == pytest.approx(100 * 1024 * 2)
    assert float(rows["dispatch"][5]) == pytest.approx(200 * 1024)
    assert float(rows["second"][4]) == pytest.approx(20 * 1024 * 2)
    assert f"row_source_hash = {rps.source_hash(rps.ROW_SOURCES)}" in md


def test_committed_row_mover_tables_name_their_sources():
    prof = os.path.join(ROOT, "profiles")
    files = [f for f in os.listdir(prof) if f.endswith("_counters.md") and f.startswith("row_movers")]
    assert len(files) == 2
    for f in files:
        lines = [l for l in open(os.path.join(prof, f)) if l.startswith("row_source_hash = ")]
        assert len(lines) == 1 and len(lines[0].split("=")[1].strip()) == 16, f
