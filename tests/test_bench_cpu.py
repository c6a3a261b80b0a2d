"""Host logic of bench.py, on the CPU: the one-GPU refusal and the counter
calibration behind roofline.traffic (no GPU, no kernel launch)."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

LOGITS = "void lce::mfma2::ring::k_ring<true, true, 0, 0>(lce::GemmDesc, long, long, long)"
GRAD_X = "void lce::mfma2::ring::k_ring<true, false, 1, 0, 4>(lce::GemmDesc, long, long, long)"
ROW_CE = "void lce::k_row_ce_pf<unsigned short, 16>(unsigned short const*, long)"
COPY = "__amd_rocclr_copyBuffer"


def _counter_dir(tmp_path, name, counter, rows):
    """A rocprofv3-style counter_collection.csv with (kernel, value) rows."""
    d = tmp_path / name / "host"
    d.mkdir(parents=True)
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (k, v) in enumerate(rows):
            w.writerow([i + 1, k, counter, v])
    return str(tmp_path / name)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def test_traffic_calibration_scales_by_the_copy_reading(tmp_path, monkeypatch):
    """Each counter is scaled by 1 GiB over its own reading for the 1 GiB
    copy; per kernel class the second half of the dispatches (the timed
    step) is averaged; traffic = fetched + written."""
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "traffic_path", lambda workload: str(out))
    kib = 1024.0
    fetch = _counter_dir(tmp_path, "fetch", "FETCH_SIZE", [
        (COPY, (1 << 29) / kib),                       # reads half of 1 GiB: factor 2
        (LOGITS, 9e6), (LOGITS, 9e6), (LOGITS, 3e6), (LOGITS, 5e6),
        (GRAD_X, 1e6), (GRAD_X, 2e6),
        ("some_other_kernel", 7.0),
    ])
    write = _counter_dir(tmp_path, "write", "WRITE_SIZE", [
        (COPY, (1 << 30) / kib),                       # factor 1
        (LOGITS, 1e6), (LOGITS, 1e6), (LOGITS, 2e6), (LOGITS, 2e6),
        (ROW_CE, 4e6), (ROW_CE, 6e6),
    ])
    bench.summarise_traffic("unit", fetch, write)
    t = json.loads(out.read_text())
    assert t["FETCH_SIZE_factor"] == pytest.approx(2.0)
    assert t["WRITE_SIZE_factor"] == pytest.approx(1.0)
    k = t["kernels"]
    assert k["logits_gemm"]["fetch_size_bytes"] == pytest.approx(4e6 * kib * 2.0)
    assert k["logits_gemm"]["write_size_bytes"] == pytest.approx(2e6 * kib)
    assert k["logits_gemm"]["traffic_bytes"] == pytest.approx(4e6 * kib * 2.0 + 2e6 * kib)
    assert k["grad_x_gemm"]["traffic_bytes"] == pytest.approx(2e6 * kib * 2.0)
    assert k["row_ce"]["traffic_bytes"] == pytest.approx(6e6 * kib)
    assert set(k) == {"logits_gemm", "grad_x_gemm", "row_ce"}
    assert t["source_hash"] == bench.kernel_source_hash()


def test_traffic_is_dropped_when_the_sources_change(tmp_path, monkeypatch):
    p = tmp_path / "t.json"
    monkeypatch.setattr(bench, "traffic_path", lambda workload: str(p))
    p.write_text(json.dumps({"source_hash": bench.kernel_source_hash(), "kernels": {}}))
    assert bench.load_traffic("unit") is not None
    p.write_text(json.dumps({"source_hash": "0" * 16, "kernels": {}}))
    assert bench.load_traffic("unit") is None


def test_source_hash_ignores_comments_and_layout():
    a = "int f(int x) {  // doubles\n  return 2 * x; /* no\n overflow */ }\n"
    b = "int f(int x) {\n    return 2 * x;\n}"
    c = "int f(int x) { return 3 * x; }"
    assert bench.code_tokens(a) == bench.code_tokens(b)
    assert bench.code_tokens(a) != bench.code_tokens(c)


def test_kernel_classes_cover_the_launched_gemms():
    """Every GEMM and row kernel of the FLCE step maps to one class."""
    names = {
        LOGITS: "logits_gemm",
        GRAD_X: "grad_x_gemm",
        "void lce::mfma2::ring::k_ring<false, false, 1, 0>(lce::GemmDesc, long, long, long)": "grad_w_gemm",
        "void lce::mfma2::ring::k_ring<false, false, 2, 0>(lce::GemmDesc, long, long, long)": "grad_w_gemm",
        "void lce::mfma2::ring::k_ring<false, false, 4, 0, 4>(lce::GemmDesc, long, long, long)": "grad_w_gemm",
        "void lce::mfma2::ring::k_ring<false, true, 2, 0, 4>(lce::GemmDesc, long, long, long)": "grad_w_gemm",
        "void lce::mfma2::ring::k_ring<true, false, 3, 0, 4>(lce::GemmDesc, long, long, long)": "grad_x_gemm",
        ROW_CE: "row_ce",
    }
    for name, kind in names.items():
        got = [k for frag, k in bench.KERNEL_KINDS.items() if frag in name]
        assert got == [kind], name


@pytest.mark.parametrize("N,H,V,dtype,chunk", [
    (32768, 4096, 128256, "bf16", 0), (8192, 2048, 128256, "bf16", 0),
    (32768, 4096, 256000, "bf16", 0), (32768, 4096, 128256, "bf16", 2048),
    (256, 64, 1024, "f32", 0), (1000, 136, 4099, "bf16", 256)])
def test_workspace_parts_and_the_one_chunk_bound(N, H, V, dtype, chunk):
    """The library's workspace regions sum to its workspace query and have the
    documented sizes, and the whole workspace is within the bench's bound:
    one chunk of logits + (N + V) x 16 bytes + the grad_X split-K partials
    (which hold the gathered rows of a packed chunk)."""
    from linear_cross_entropy_03_amd import binding as B
    dt = B.BF16 if dtype == "bf16" else B.F32
    e = 2 if dtype == "bf16" else 4
    up = lambda x: (x + 255) // 256 * 256
    c, s = B.flce_plan(N, H, V, dt, chunk)
    ws = B.flce_workspace_bytes(N, H, V, dt, chunk)
    parts = bench.scratch_parts(B, N, H, V, dt, chunk)
    assert set(parts) == {"rows", "chunk_logits", "split_partials", "pack_lists", "workspace"}
    assert parts["workspace"] == ws
    assert parts["chunk_logits"] == up(c * ((V + 7) // 8 * 8) * e)
    if e == 2:
        assert parts["split_partials"] >= up(c * H * 4)      # room for the gathered rows too
    assert parts["rows"] <= 256 + up(4 * N) and parts["pack_lists"] <= 3 * up(4 * N) + 4096
    assert ws <= bench.one_chunk_bound_bytes(parts, N, V)
